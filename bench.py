#!/usr/bin/env python3
"""Decode benchmark of the CSA / HCA hybrid attention hot path on one MI355X.

Workload (the 1M-context configuration): an interleaved stack of 8 attention
layers, CSA (m = 4, two-path compression, Lightning Indexer with 64 heads x
128, top-1024, 128-token window, sinks) alternating with HCA (m = 128, dense,
128-token window, sinks); 64 query heads x d = 512 sharing one KV head; bf16
storage, fp32 accumulation; n_ctx = 1,000,000 tokens; batch 16.  All eight
layers' compressed caches are resident in HBM (about 2.4 GB per sequence).

One step decodes the token at position t = n_ctx - 1 of every sequence
through all 8 layers, with the decode-time maintenance of the caches: on a
second stream csa_window_append puts the token's raw K/V rows into every
layer's window ring and csa_compress_append stages its compression inputs,
writing the entry whose block it completes (every CSA step at t = 999,999; HCA
blocks complete every 128th token); per CSA layer the indexer scores every
visible entry and keeps the top 1024 (csa_index_topk: one scan kernel that
also selects each part's candidates, then a merge kernel) and
csa_sparse_attn attends over them plus the window; per HCA layer
hca_dense_attn attends over all 7812 visible entries plus the window.

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


# Layer schedules of the stack (trdm.cn, section 4.3, the layer-interleaving
# paragraph): CSA and HCA alternate; V4-Flash-style stacks open with two
# layers of sliding-window attention only, V4-Pro-style ones with two HCA
# layers.
SCHEDULES = ("alternate", "flash", "pro", "csa", "hca")


class Stack:
    """Shapes of the 8-layer decode workload and its algorithmic bytes."""

    def __init__(self, B=16, n_ctx=1_000_000, layers=8, eb=2, schedule="alternate", W=128, index_fmt=None):
        assert schedule in SCHEDULES and index_fmt in (None, "mxfp4")
        self.B, self.n_ctx, self.layers, self.schedule = B, n_ctx, layers, schedule
        self.eb = eb  # bytes per stored element: caches, window, indexer q/k, compression inputs
        # "mxfp4": the indexer's q and keys are MXFP4 (E2M1 + one E8M0 scale per
        # 32 elements: 17/32 B per element), its raw key rows bf16, and the
        # appends compress them straight to MXFP4 entries
        self.ix = index_fmt
        self.ieb = 17 / 32 if index_fmt == "mxfp4" else eb
        self.H, self.d = 64, 512
        self.HI, self.dI = 64, 128
        self.k, self.W = 1024, W
        self.m_csa, self.m_hca = 4, 128
        self.L_csa = -(-n_ctx // self.m_csa)
        self.L_hca = -(-n_ctx // self.m_hca)
        self.t = n_ctx - 1  # the token each step decodes (the last of the history)
        self.nv_csa = min(self.L_csa, self.t // self.m_csa)
        self.nv_hca = min(self.L_hca, self.t // self.m_hca)
        self.scale = 1.0 / math.sqrt(self.d)

    def kinds(self):
        if self.schedule in ("csa", "hca"):  # one layer kind throughout (the single-layer configurations)
            return [self.schedule] * self.layers
        alt = ["csa" if i % 2 == 0 else "hca" for i in range(self.layers)]
        if self.schedule == "flash":
            return ["win", "win"] + alt[:self.layers - 2]
        if self.schedule == "pro":
            return ["hca", "hca"] + alt[:self.layers - 2]
        return alt

    def emits(self, m):
        """Whether the decoded token completes its block (an entry is written)."""
        return (self.t + 1) % m == 0

    # ---- algorithmic bytes (what the method must move), per query ----------
    def index_bytes(self):
        """csa_index_topk per query: the visible indexer keys, the query's
        index heads and head weights, the selected indices written."""
        return self.nv_csa * self.dI * self.ieb + self.HI * self.dI * self.ieb + self.HI * 4 + self.k * 4

    def _append_bytes(self, D, streams, m, e_in=None, e_out=None):
        """csa_compress_append of one stream: the new token's rows read and
        staged, and when its block completes the block's rows (and the
        previous block's, two-path) read and the entry written."""
        e = self.eb if e_in is None else e_in
        b = 2 * streams * D * e
        if self.emits(m):
            b += streams * m * D * e + D * (e if e_out is None else e_out)
        return b

    def _window_bytes(self):
        """Attention's raw window rows, and csa_window_append of the new token."""
        e = self.eb
        return (self.W * self.d * 2 * e + 2 * 2 * self.d * e) if self.W else 0

    def csa_bytes(self):
        b = self.index_bytes()
        e = self.eb
        b += self.k * self.d * 2 * e            # gathered compressed K and V rows
        b += self._window_bytes()
        b += 2 * self.H * self.d * 2            # q and out (bf16)
        b += self.k * 4                         # selected indices, read by the attention
        for D in (self.d, self.d):              # K and V, two-path (4 streams)
            b += self._append_bytes(D, 4, self.m_csa)
        if self.ix == "mxfp4":                  # index keys: bf16 rows in, MXFP4 entries out
            b += self._append_bytes(self.dI, 4, self.m_csa, 2, self.ieb)
        else:
            b += self._append_bytes(self.dI, 4, self.m_csa)
        return b

    def hca_bytes(self):
        e = self.eb
        b = self.nv_hca * self.d * 2 * e + self._window_bytes() + 2 * self.H * self.d * 2
        for D in (self.d, self.d):              # K and V, single path (2 streams)
            b += self._append_bytes(D, 2, self.m_hca)
        return b

    def win_bytes(self):
        return self._window_bytes() + 2 * self.H * self.d * 2

    def layer_bytes(self, kind):
        return {"csa": self.csa_bytes, "hca": self.hca_bytes, "win": self.win_bytes}[kind]()

    def step_bytes(self):
        return sum(self.layer_bytes(k) for k in self.kinds()) * self.B


def raw_rows(st: Stack, name, layer, p0, cnt, D, device, scale, dtype=torch.bfloat16):
    """Rows p0 .. p0+cnt-1 of a virtual raw stream [B][n_ctx][D]."""
    b = torch.arange(st.B, dtype=torch.int64, device=device).reshape(-1, 1)
    p = torch.arange(p0, p0 + cnt, dtype=torch.int64, device=device).reshape(1, -1)
    r = (b * st.n_ctx + p).reshape(-1)
    return syn.rows((st.B, st.n_ctx, D), r, SEED, syn.TID[name], dtype=dtype, device=device,
                    scale=scale, layer=layer).reshape(st.B, cnt, D)


def ring_of(rows, p0):
    """Rows of positions p0 .. p0+S-1 ([B][S][D]) placed at ring slots u % S."""
    S = rows.shape[1]
    out = torch.empty_like(rows)
    out[:, torch.arange(p0, p0 + S, device=rows.device) % S] = rows
    return out


# Raw-stream names of the compressed streams: (value A, logits A, value B, logits B).
STREAMS = {"k": ("k", "z_k", "xb_k", "zb_k"), "v": ("v", "z_v", "xb_v", "zb_v"),
           "idx": ("k_idx", "z_idx", "xb_idx", "zb_idx")}


# E8M0 scales of the generated MXFP4 indexer tensors: 2^-2 .. 2^2
MX_SCALES = (125, 129)


def mxfp4_tensor(shape, name, layer, device):
    """A seeded MXFP4 tensor of logical shape `shape` (random E2M1 codes,
    E8M0 scales in MX_SCALES), wrapped for the binding."""
    import compressed_sparse_kv_compress_amd as csa
    n = math.prod(shape)
    buf = syn.mxfp4_(torch.empty(n // 2 + n // 32, dtype=torch.uint8, device=device), SEED, syn.TID[name], n,
                     scale_lo=MX_SCALES[0], scale_hi=MX_SCALES[1], layer=layer)
    return csa.MXFP4(buf, shape)


class GpuState:
    """All device buffers of the workload, generated in place on the GPU, and
    the decode step over them."""

    def __init__(self, st: Stack, device="cuda"):
        """st.eb == 2: bf16 storage.  st.eb == 1: FP8 (E4M3) storage of the
        caches, the window, the indexer's q and keys and the compression
        inputs; the attention query and output stay bf16.  FP8 K/V rows are
        unit-scale codes with the K scale 1/sqrt(d) folded into the softmax
        scale (the V scale would fold into the output's consumer).

        The caches hold the history (generated directly); the raw rows of the
        decoded token and of the earlier tokens of its block(s) sit in the
        per-stream staging rings and the new-token rows, the last W raw
        positions in the window rings (slot = position % W)."""
        import compressed_sparse_kv_compress_amd as csa
        self.csa = csa
        self.st = st
        bf = torch.bfloat16
        sto = bf if st.eb == 2 else torch.float8_e4m3fn
        B, d, dI, H, W, t = st.B, st.d, st.dI, st.H, st.W, st.t
        si = dI ** -0.5
        sd = d ** -0.5 if st.eb == 2 else 1.0          # K/V value scale
        self.ascale = st.scale if st.eb == 2 else st.scale * d ** -0.5
        self.pos = torch.full((B,), t, dtype=torch.int64, device=device)
        self.ring_layout = csa.layout(ring=True)
        self.layers = []
        for li, kind in enumerate(st.kinds()):
            lay = {"kind": kind}

            def gen(shape, name, scale, dtype=bf, li=li):
                x = torch.empty(shape, dtype=dtype, device=device)
                return syn.fill_(x, SEED, syn.TID[name], scale=scale, layer=li)

            lay["q"] = gen((B, 1, H, d), "q", d ** -0.5)
            lay["sink"] = gen((H,), "sink", 1.0, torch.float32)
            if W:
                lay["kr"] = ring_of(raw_rows(st, "kr", li, t - W + 1, W, d, device, sd, sto), t - W + 1)
                lay["vr"] = ring_of(raw_rows(st, "vr", li, t - W + 1, W, d, device, sd, sto), t - W + 1)
                lay["k_new"] = raw_rows(st, "kr", li, t, 1, d, device, sd, sto)[:, 0].contiguous()
                lay["v_new"] = raw_rows(st, "vr", li, t, 1, d, device, sd, sto)[:, 0].contiguous()
            else:
                lay["kr"] = lay["vr"] = None
            lay["out"] = torch.empty((B, 1, H, d), dtype=bf, device=device)
            if kind == "csa":
                m, S = st.m_csa, 2 * st.m_csa
                L = st.L_csa
                lay["kc"] = gen((B, L, d), "kc", sd, sto)
                lay["vc"] = gen((B, L, d), "vc", sd, sto)
                if st.ix == "mxfp4":
                    lay["ki"] = mxfp4_tensor((B, L, dI), "kic", li, device)
                    lay["qi"] = mxfp4_tensor((B, 1, st.HI, dI), "q_idx", li, device)
                else:
                    lay["ki"] = gen((B, L, dI), "kic", si, sto)
                    lay["qi"] = gen((B, 1, st.HI, dI), "q_idx", si, sto)
                lay["wi"] = gen((B, 1, st.HI), "w_idx", st.HI ** -0.5, torch.float32)
                for s, D, sc in (("k", d, sd), ("v", d, sd), ("idx", dI, si)):
                    scales = (sc, 0.5, sc, 0.5)
                    rdt = bf if (s == "idx" and st.ix == "mxfp4") else sto
                    lay["new_" + s] = [raw_rows(st, nm, li, t, 1, D, device, scl, rdt)[:, 0].contiguous()
                                       for nm, scl in zip(STREAMS[s], scales)]
                    lay["ring_" + s] = [ring_of(raw_rows(st, nm, li, t - S + 1, S, D, device, scl, rdt), t - S + 1)
                                        for nm, scl in zip(STREAMS[s], scales)]
                lay["idx"] = torch.empty((B, 1, st.k), dtype=torch.int32, device=device)
                lay["itk_ws"] = torch.zeros(max(16, csa.csa_index_topk_workspace(B, 1, L, st.HI, st.k)),
                                            dtype=torch.uint8, device=device)
                nb = csa.csa_attn_workspace(B, 1, H, d, st.k + W)
            elif kind == "hca":
                m = S = st.m_hca
                L = st.L_hca
                lay["kc"] = gen((B, L, d), "kc", sd, sto)
                lay["vc"] = gen((B, L, d), "vc", sd, sto)
                for s in ("k", "v"):
                    names = (s, "z_" + s)
                    lay["new_" + s] = [raw_rows(st, nm, li, t, 1, d, device, scl, sto)[:, 0].contiguous()
                                       for nm, scl in zip(names, (sd, 0.5))]
                    lay["ring_" + s] = [ring_of(raw_rows(st, nm, li, t - S + 1, S, d, device, scl, sto), t - S + 1)
                                        for nm, scl in zip(names, (sd, 0.5))]
                nb = csa.csa_attn_workspace(B, 1, H, d, st.nv_hca + W)
            else:  # sliding window only: no compressed cache
                lay["kc"] = torch.empty((B, 0, d), dtype=sto, device=device)
                lay["vc"] = torch.empty((B, 0, d), dtype=sto, device=device)
                nb = csa.csa_attn_workspace(B, 1, H, d, W)
            lay["ws"] = torch.empty(max(nb, 16), dtype=torch.uint8, device=device)
            self.layers.append(lay)
        self.side = torch.cuda.Stream(device=device)  # default priority
        torch.cuda.synchronize()

    def step(self, ev=None, only=None, csa_layer=None, scan_ev=None):
        """One decode step of the token at t = n_ctx - 1 through all layers.

        The side stream first appends the token's raw window rows to every
        layer's window ring (joined before the first attention), then its
        compression inputs to the staging rings, writing the entry whose block
        it completes; that entry is not visible to the token itself, so
        attention never waits for compression.  The main stream runs, per
        CSA layer, the indexer + top-k and the sparse attention, per HCA
        layer the dense attention, per window layer the window attention.
        ev: optional dict of event lists keyed by call name; events bracket
        calls (all, or the names in `only`) on the stream that runs them;
        csa_layer: bracket only that CSA layer's index call (every timing
        event costs a few microseconds of idle GPU between kernels);
        scan_ev: (CSA layer, (start, stop)): that layer's scan kernel records
        the two events itself as it starts and ends (no idle gap)."""
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

        with torch.cuda.stream(side):
            mark("window_append")
            for lay in self.layers:
                if lay["kr"] is not None:
                    csa.csa_window_append(lay["k_new"], lay["v_new"], lay["kr"], lay["vr"], self.pos)
            mark("window_append_end")
            windows = torch.cuda.Event()
            windows.record()
            for lay in self.layers:
                if lay["kind"] == "csa":
                    mark("csa_compress")
                    for s, cache in (("k", "kc"), ("v", "vc"), ("idx", "ki")):
                        xa, za, xb, zb = lay["new_" + s]
                        csa.csa_compress_append(xa, za, st.m_csa, lay["ring_" + s], self.pos, lay[cache], x_b=xb,
                                                z_b=zb)
                    mark("csa_compress_end")
                elif lay["kind"] == "hca":
                    mark("hca_compress")
                    for s, cache in (("k", "kc"), ("v", "vc")):
                        x, z = lay["new_" + s]
                        csa.csa_compress_append(x, z, st.m_hca, lay["ring_" + s], self.pos, lay[cache])
                    mark("hca_compress_end")

        ci = 0
        joined = False
        for lay in self.layers:
            if lay["kind"] == "csa":
                mark("index_topk", ci)
                if scan_ev is not None and scan_ev[0] == ci:
                    csa.time_next_scan(*scan_ev[1])
                csa.csa_index_topk(lay["qi"], lay["ki"], st.m_csa, st.k, w_idx=lay["wi"], n_ctx=st.n_ctx,
                                   idx=lay["idx"], ws=lay["itk_ws"])
                mark("index_topk_end", ci)
                ci += 1
            if not joined:
                main.wait_event(windows)
                joined = True
            if lay["kind"] == "csa":
                mark("csa_sparse_attn")
                csa.csa_sparse_attn(lay["q"], lay["kc"], lay["vc"], lay["idx"], kr=lay["kr"], vr=lay["vr"],
                                    W=st.W, sink=lay["sink"], scale=self.ascale, n_ctx=st.n_ctx, out=lay["out"],
                                    ws=lay["ws"], layout=self.ring_layout)
                mark("csa_sparse_attn_end")
            elif lay["kind"] == "hca":
                mark("hca_dense_attn")
                csa.hca_dense_attn(lay["q"], lay["kc"], lay["vc"], st.m_hca, kr=lay["kr"], vr=lay["vr"], W=st.W,
                                   sink=lay["sink"], scale=self.ascale, n_ctx=st.n_ctx, out=lay["out"],
                                   ws=lay["ws"], layout=self.ring_layout)
                mark("hca_dense_attn_end")
            else:
                mark("window_attn")
                csa.hca_dense_attn(lay["q"], lay["kc"], lay["vc"], st.m_hca, kr=lay["kr"], vr=lay["vr"], W=st.W,
                                   sink=lay["sink"],
                                   scale=self.ascale, n_ctx=st.n_ctx, out=lay["out"], ws=lay["ws"],
                                   layout=self.ring_layout)
                mark("window_attn_end")
        main.wait_stream(side)

    def capture(self, steps: int = 1):
        """`steps` consecutive decode steps as one HIP graph (stream-ordered
        capture of the same calls on both streams, each step joined before
        the next as in eager order); returns a callable that replays it.  A
        serving loop replays several steps per launch to spread the graph's
        launch cost."""
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.step()  # warm the allocator and the kernels outside the graph
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(steps):
                self.step()
        torch.cuda.synchronize()
        return g.replay


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
                      for f in ("index.hip", "topk.hip", "select.hpp", "merge.hpp", "kernels.hpp", "common.hpp")]


def source_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel_src, per_launch_units, key="hbm_bytes_per_launch"):
    """HBM bytes per csa_index_topk call (its two kernels; key names the scan
    kernel alone with index_score_stream_hbm_bytes_per_launch) from the
    committed rocprofv3 counter summary, or None when it is missing or the
    kernels' sources changed since."""
    path = os.path.join(ROOT, "profiles", "index_topk_stack8_b16_counters.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"^source_sha256_16:\s*(\w+)", txt, re.M)
    m_b = re.search(r"^" + key + r":\s*([0-9.eE+]+)", txt, re.M)
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

    sub = Stack(B=S, n_ctx=st.n_ctx, layers=st.layers, schedule=st.schedule)
    per_layer = min_seconds / st.layers
    step_s, total, reps_all = 0.0, 0.0, []
    for li, kind in enumerate(st.kinds()):
        t_layer, reps = _oracle_layer(st, sub, S, full, sd, si, li, kind, per_layer, max_reps)
        step_s += t_layer / reps
        total += t_layer
        reps_all.append(reps)
        print("# cpu oracle: layer %d (%s) %.2f s over %d repetition(s)" % (li, kind, t_layer, reps),
              file=sys.stderr, flush=True)
    threads = int(os.environ.get("OMP_NUM_THREADS", host_cores()))
    return {"value": S / step_s, "unit": "queries/s", "cores": min(S, threads, host_cores()), "kind": "oracle",
            "host_cores": host_cores(),
            "sample": "%d of %d sequences, one decode step through all %d layers, each layer's oracle calls "
                      "repeated %s times on the same inputs (%.1f s of oracle time); the oracle runs one "
                      "OpenMP thread per (sequence, query)" % (S, st.B, st.layers, "/".join(map(str, reps_all)), total)}


def host_cores():
    """Host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _oracle_layer(st, sub, S, full, sd, si, li, kind, min_seconds, max_reps):
    """Oracle calls of one layer of the decode step for S sequences, repeated
    until min_seconds (at most max_reps times); returns (seconds, repetitions),
    input regeneration excluded."""
    import numpy as np

    import oracle
    L = {"csa": st.L_csa, "hca": st.L_hca, "win": 0}[kind]
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
        e = st.t // m  # the entry the decoded token completes (when it does)
        p0 = (e - 1) * m
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
                if st.emits(m):
                    oracle.compress(xa, za, m, x_b=xb, z_b=zb, n=st.n_ctx, p0=p0, e0=e, e1=e + 1)
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
    else:  # HCA, or window only (no compressed entries)
        m = st.m_hca
        e = st.t // m
        p0 = e * m
        raws = [raw_rows(sub, nm, li, p0, m, st.d, "cpu", scl).double().numpy()
                for nm, scl in (("k", sd), ("z_k", 0.5), ("v", sd), ("z_v", 0.5))] if kind == "hca" else None
        kc = np.stack([full((st.B, L, st.d), "kc", sd, li, rows=seq_rows(b, L)) for b in range(S)]) if L else \
            np.zeros((S, 0, st.d))
        vc = np.stack([full((st.B, L, st.d), "vc", sd, li, rows=seq_rows(b, L)) for b in range(S)]) if L else \
            np.zeros((S, 0, st.d))
        while reps < max_reps and (reps == 0 or total < min_seconds):
            reps += 1
            t0 = time.perf_counter()
            if raws is not None and st.emits(m):
                oracle.compress(raws[0], raws[1], m, n=st.n_ctx, p0=p0, e0=e, e1=e + 1)
                oracle.compress(raws[2], raws[3], m, n=st.n_ctx, p0=p0, e0=e, e1=e + 1)
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


def fp8_storage_step(B: int, steps: int, warmup: int, index_fmt=None):
    """The same 8-layer decode step with FP8 (E4M3) storage: reported beside
    the bf16 headline, never as it.  index_fmt "mxfp4": the pages' own mix,
    FP8 main KV with the indexer's q.k in FP4 (MXFP4 q and keys, the appends
    compressing bf16 index-key rows straight to MXFP4 entries)."""
    st = Stack(B=B, eb=1, index_fmt=index_fmt)
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
        "storage": ("E4M3 K/V caches, window and K/V compression inputs; MXFP4 indexer q and keys (bf16 index-key "
                    "rows compressed to MXFP4 by the appends); bf16 query and output" if index_fmt else
                    "E4M3 caches, window, indexer q/k and compression inputs; bf16 query and output"),
        "ms_per_step": ms, "queries_per_s": st.B / (ms * 1e-3),
        "algorithmic_bytes_per_step": st.step_bytes(),
        "achieved_GBps": st.step_bytes() / (ms * 1e-3) / 1e9,
        "index_topk_GBps": idx_bytes / (per_call["index_topk"] * 1e-3) / 1e9,
        "per_call_ms": per_call,
        "note": "attention converts each E4M3 row to bf16 before the bf16 MFMA sequence; at B=16 the decode "
                "attention kernels are bound by their per-stage chain, not by bytes, so the gain comes "
                "from the indexer scan",
    }


def prefill_index_topk(queries: int = 4096, reps: int = 3, fp8: bool = False, mxfp4: bool = False):
    """csa_index_topk on the CSA prefill-chunk shape: the last `queries` of a
    65,536-token chunk after a 262,144-token prefix (81,920 compressed
    entries, about 82 K visible per query), 64 index heads x 128, k = 1024;
    bf16, E4M3 query and keys (the same values rounded to E4M3), or MXFP4
    (random E2M1 codes, E8M0 scales 2^-2 .. 2^2)."""
    import compressed_sparse_kv_compress_amd as csa
    HI, dI, m, k = 64, 128, 4, 1024
    prefix, chunk = 262144, 65536
    n_ctx = prefix + chunk
    L = n_ctx // m
    ki = syn.fill_(torch.empty((1, L, dI), dtype=torch.bfloat16, device="cuda"), 4, syn.TID["kic"], scale=dI ** -0.5)
    qi = syn.fill_(torch.empty((1, queries, HI, dI), dtype=torch.bfloat16, device="cuda"), 4, syn.TID["q_idx"],
                   scale=dI ** -0.5)
    if fp8:
        ki, qi = ki.to(torch.float8_e4m3fn), qi.to(torch.float8_e4m3fn)
    if mxfp4:
        del ki, qi
        nq, nk = queries * HI * dI, L * dI
        qb = syn.mxfp4_(torch.empty(nq // 2 + nq // 32, dtype=torch.uint8, device="cuda"), 4, syn.TID["q_idx"], nq,
                        scale_lo=125, scale_hi=129)
        kb = syn.mxfp4_(torch.empty(nk // 2 + nk // 32, dtype=torch.uint8, device="cuda"), 4, syn.TID["kic"], nk,
                        scale_lo=125, scale_hi=129)
        qi, ki = csa.MXFP4(qb, (1, queries, HI, dI)), csa.MXFP4(kb, (1, L, dI))
    wi = syn.fill_(torch.empty((1, queries, HI), device="cuda"), 4, syn.TID["w_idx"], scale=HI ** -0.5)
    ws = torch.zeros(csa.csa_index_topk_workspace(1, queries, L, HI, k), dtype=torch.uint8, device="cuda")
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
    peak = 10100.0 if mxfp4 else (5000.0 if fp8 else 2500.0)
    return {"queries": queries, "entries": L, "storage": "mxfp4" if mxfp4 else ("e4m3" if fp8 else "bf16"),
            "ms_per_call": ms,
            "tflops": flop / (ms * 1e-3) / 1e12, "peak_tflops": peak, "frac_of_peak": flop / (ms * 1e-3) / 1e12 / peak,
            "visible_pairs": pairs,
            "note": "flop = 2 * visible (query, entry) pairs * index heads * index dim, against the dense MFMA peak "
                    "of the storage type; scores by the 16-row prefill kernel (each key tile read once per 16 "
                    "queries), then the stand-alone top-k (about a sixth of the bf16 call)"}


GRAPH_STEPS = 8  # decode steps per graph in the multi-step replay


def timed_steps(run, steps, warmup):
    """Average ms per call of run() over `steps` calls after `warmup`."""
    for _ in range(warmup):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def decode_step_b1(steps: int, warmup: int, schedule: str = "alternate"):
    """The same bf16 8-layer step for one sequence (B = 1): the latency-bound
    end of the decode workload, reported beside the B = 16 headline, eager
    and as one HIP-graph replay per step."""
    st = Stack(B=1, schedule=schedule)
    state = GpuState(st)
    ms = timed_steps(state.step, steps, warmup)
    replay = state.capture()
    ms_graph = timed_steps(replay, steps, warmup)
    replay8 = state.capture(GRAPH_STEPS)
    ms_graph8 = timed_steps(replay8, max(1, steps // GRAPH_STEPS), 1) / GRAPH_STEPS
    ev = {}
    for _ in range(3):
        state.step(ev)
    torch.cuda.synchronize()
    per_call = event_means_ms(ev)
    del state, replay, replay8
    torch.cuda.empty_cache()
    best = min(ms, ms_graph, ms_graph8)
    return {"ms_per_step": ms, "graph_ms_per_step": ms_graph, "graph8_ms_per_step": ms_graph8,
            "tokens_per_s": 1.0 / (best * 1e-3),
            "algorithmic_bytes_per_step": st.step_bytes(),
            "achieved_GBps": st.step_bytes() / (best * 1e-3) / 1e9, "per_call_ms": per_call,
            "note": "one query per call: bound by the latency of the calls' kernels; the graph replays submit the "
                    "whole step (both streams), or %d consecutive steps, at once; rates use the fastest" % GRAPH_STEPS}


def schedules_b16(steps: int, warmup: int, B: int):
    """The step under the V4-Flash- and V4-Pro-style layer schedules."""
    res = {}
    for sch in ("flash", "pro"):
        st = Stack(B=B, schedule=sch)
        state = GpuState(st)
        ms = timed_steps(state.step, steps, warmup)
        del state
        torch.cuda.empty_cache()
        res[sch] = {"layers": st.kinds(), "ms_per_step": ms, "queries_per_s": st.B / (ms * 1e-3),
                    "algorithmic_bytes_per_step": st.step_bytes(),
                    "achieved_GBps": st.step_bytes() / (ms * 1e-3) / 1e9}
    return res


def single_layer_decode(steps, warmup, kind, B, n_ctx, W):
    """Decode of one layer (configurations 2 and 3): the same step machinery
    with one CSA or one HCA layer; queries/s and algorithmic bytes."""
    st = Stack(B=B, n_ctx=n_ctx, layers=1, schedule=kind, W=W)
    state = GpuState(st)
    ms = timed_steps(state.step, steps, warmup)
    replay = state.capture()
    ms_graph = timed_steps(replay, steps, warmup)
    replay8 = state.capture(GRAPH_STEPS)
    ms_graph8 = timed_steps(replay8, max(1, steps // GRAPH_STEPS), 1) / GRAPH_STEPS
    ev = {}
    for _ in range(3):
        state.step(ev)
    torch.cuda.synchronize()
    per_call = event_means_ms(ev)
    del state, replay, replay8
    torch.cuda.empty_cache()
    best = min(ms, ms_graph, ms_graph8)
    gbps = st.step_bytes() / (best * 1e-3) / 1e9
    return {"batch": B, "n_ctx": n_ctx, "layer": kind, "window": W, "ms_per_step": ms, "graph_ms_per_step": ms_graph,
            "graph8_ms_per_step": ms_graph8,
            "queries_per_s": B / (best * 1e-3), "algorithmic_bytes_per_step": st.step_bytes(), "achieved_GBps": gbps,
            "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS, "per_call_ms": per_call,
            "note": "a few launches per step: bound by launch latency; rates use the fastest of eager launches, one "
                    "HIP-graph replay per step, and one replay of %d consecutive steps (both streams)" % GRAPH_STEPS}


def bulk_compress(kind, B, n, reps=3):
    """Bulk (prefill) compression of whole raw streams: CSA two-path (m = 4)
    of the K, V and index-key streams of configuration 2, or HCA (m = 128) of
    the K and V streams of configuration 3.  Bytes: every raw value and logit
    read once, every entry written once."""
    import compressed_sparse_kv_compress_amd as csa
    m = 4 if kind == "csa" else 128
    dims = (512, 512, 128) if kind == "csa" else (512, 512)
    total_bytes, total_ms = 0, 0.0
    for si, D in enumerate(dims):
        arrs = [syn.fill_(torch.empty((B, n, D), dtype=torch.bfloat16, device="cuda"), 2, 30 + 4 * si + j,
                          scale=0.5 if j % 2 else D ** -0.5) for j in range(4 if kind == "csa" else 2)]
        L = -(-n // m)
        out = torch.empty((B, L, D), dtype=torch.bfloat16, device="cuda")
        if kind == "csa":
            call = lambda: csa.csa_compress(arrs[0], arrs[1], m, x_b=arrs[2], z_b=arrs[3], out=out)  # noqa: E731
        else:
            call = lambda: csa.hca_compress(arrs[0], arrs[1], m, out=out)  # noqa: E731
        total_ms += timed_steps(call, reps, 1)
        total_bytes += sum(a.numel() for a in arrs) * 2 + out.numel() * 2
        if kind == "csa" and D == 128:  # the index keys again, written as MXFP4 entries
            nel = B * L * D
            mx = csa.MXFP4(torch.empty(nel // 2 + nel // 32, dtype=torch.uint8, device="cuda"), (B, L, D))
            mx_ms = timed_steps(lambda: csa.csa_compress(arrs[0], arrs[1], m, x_b=arrs[2], z_b=arrs[3], out=mx),
                                reps, 1)
            mx_bytes = sum(a.numel() for a in arrs) * 2 + mx.data.numel()
            mx_entry = {"ms": mx_ms, "bytes": mx_bytes, "GBps": mx_bytes / (mx_ms * 1e-3) / 1e9,
                        "bf16_out_ms": timed_steps(call, reps, 1)}
            del mx
        del arrs, out
        torch.cuda.empty_cache()
    gbps = total_bytes / (total_ms * 1e-3) / 1e9
    res = {"batch": B, "tokens": n, "m": m, "streams": len(dims), "ms": total_ms, "bytes": total_bytes,
           "GBps": gbps, "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS,
           "bytes_per_sequence": total_bytes / B}
    if kind == "csa":
        res["index_keys_mxfp4"] = mx_entry
    return res


def paged_layout(B: int = 16, n_ctx: int = 1_000_000, page: int = 64, reps: int = 10):
    """csa_index_topk and csa_sparse_attn of one CSA layer over a serving
    layout: per-sequence lengths (n_ctx, n_ctx - 37,000, n_ctx - 74,000, ...
    down the batch) and compressed caches held as pools of 64-entry pages at
    seeded random places, against the same calls on dense [B][L] caches with
    the same lengths.  The outputs must agree bit for bit (they are checked
    here too); the rates count the visible index keys and gathered rows."""
    import compressed_sparse_kv_compress_amd as csa
    HI, dI, H, d, m, k, W = 64, 128, 64, 512, 4, 1024, 128
    L = -(-n_ctx // m)
    lens_l = [n_ctx - 37_000 * b for b in range(B)]
    lens = torch.tensor(lens_l, dtype=torch.int64, device="cuda")
    bf = torch.bfloat16

    def gen(shape, tid, scale, dtype=bf):
        return syn.fill_(torch.empty(shape, dtype=dtype, device="cuda"), 6, tid, scale=scale)

    ki = gen((B, L, dI), syn.TID["kic"], dI ** -0.5)
    qi = gen((B, 1, HI, dI), syn.TID["q_idx"], dI ** -0.5)
    wi = gen((B, 1, HI), syn.TID["w_idx"], HI ** -0.5, torch.float32)
    P = -(-L // page)
    npages = B * P + 8
    perm = torch.randperm(npages, generator=torch.Generator().manual_seed(6))[:B * P].reshape(B, P)
    bt = perm.to(torch.int32).cuda()
    pool = torch.empty((npages * page, dI), dtype=bf, device="cuda")
    for b in range(B):  # page p of sequence b -> pool page bt[b][p]
        rows = (bt[b].to(torch.int64).reshape(P, 1) * page + torch.arange(page, device="cuda")).reshape(-1)[:L]
        pool[rows] = ki[b]
    lay_d = csa.layout(seq_len=lens)
    lay_p = csa.layout(seq_len=lens, block_table=bt, page=page, num_pages=npages)
    ws = torch.zeros(csa.csa_index_topk_workspace(B, 1, L, HI, k), dtype=torch.uint8, device="cuda")
    idx_d = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    idx_p = torch.empty_like(idx_d)
    run_d = lambda: csa.csa_index_topk(qi, ki, m, k, w_idx=wi, n_ctx=n_ctx, layout=lay_d, idx=idx_d, ws=ws)  # noqa: E731
    run_p = lambda: csa.csa_index_topk(qi, pool, m, k, w_idx=wi, n_ctx=n_ctx, layout=lay_p, L=L, idx=idx_p,  # noqa: E731
                                       ws=ws)
    ms_d = ms_p = float("inf")
    for _ in range(3):  # alternate the two layouts; the best of three runs each
        ms_d = min(ms_d, timed_steps(run_d, reps, 2))
        ms_p = min(ms_p, timed_steps(run_p, reps, 2))
    same_idx = bool(torch.equal(idx_d, idx_p))
    vis = sum(min(L, (n - 1) // m) for n in lens_l)
    idx_bytes = vis * dI * 2 + B * (HI * dI * 2 + HI * 4 + k * 4)
    del ki, pool, ws
    torch.cuda.empty_cache()
    # sparse attention over the selection, K and V paged the same way
    kc = gen((B, L, d), syn.TID["kc"], d ** -0.5)
    vc = gen((B, L, d), syn.TID["vc"], d ** -0.5)
    q = gen((B, 1, H, d), syn.TID["q"], d ** -0.5)
    kr = gen((B, W, d), syn.TID["kr"], d ** -0.5)
    vr = gen((B, W, d), syn.TID["vr"], d ** -0.5)
    sink = gen((H,), syn.TID["sink"], 1.0, torch.float32)
    pk = torch.empty((npages * page, d), dtype=bf, device="cuda")
    pv = torch.empty_like(pk)
    for b in range(B):
        rows = (bt[b].to(torch.int64).reshape(P, 1) * page + torch.arange(page, device="cuda")).reshape(-1)[:L]
        pk[rows] = kc[b]
        pv[rows] = vc[b]
    aws = torch.empty(max(16, csa.csa_attn_workspace(B, 1, H, d, k + W)), dtype=torch.uint8, device="cuda")
    o_d = torch.empty((B, 1, H, d), dtype=bf, device="cuda")
    o_p = torch.empty_like(o_d)
    att_d = lambda: csa.csa_sparse_attn(q, kc, vc, idx_d, kr=kr, vr=vr, W=W, sink=sink, n_ctx=n_ctx,  # noqa: E731
                                        layout=lay_d, out=o_d, ws=aws)
    att_p = lambda: csa.csa_sparse_attn(q, pk, pv, idx_d, kr=kr, vr=vr, W=W, sink=sink, n_ctx=n_ctx,  # noqa: E731
                                        layout=lay_p, L=L, out=o_p, ws=aws)
    am_d = am_p = float("inf")
    for _ in range(3):
        am_d = min(am_d, timed_steps(att_d, reps, 2))
        am_p = min(am_p, timed_steps(att_p, reps, 2))
    same_out = bool(torch.equal(o_d, o_p))
    att_bytes = B * ((k + W) * d * 2 * 2 + 2 * H * d * 2 + k * 4)
    del kc, vc, pk, pv, aws
    torch.cuda.empty_cache()
    return {"batch": B, "page": page, "seq_len": lens_l,
            "index_topk": {"dense_ms": ms_d, "paged_ms": ms_p, "bytes": idx_bytes,
                           "dense_GBps": idx_bytes / (ms_d * 1e-3) / 1e9,
                           "paged_GBps": idx_bytes / (ms_p * 1e-3) / 1e9, "identical": same_idx},
            "csa_sparse_attn": {"dense_ms": am_d, "paged_ms": am_p, "bytes": att_bytes,
                                "dense_GBps": att_bytes / (am_d * 1e-3) / 1e9,
                                "paged_GBps": att_bytes / (am_p * 1e-3) / 1e9, "identical": same_out}}


def measured_peaks():
    """A plain 4 GiB device copy (read + write bytes / time) and a large bf16
    GEMM through torch (hipBLASLt): the measured counterparts of the 8 TB/s
    and 2.5 PFLOP/s spec peaks."""
    src = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = timed_steps(lambda: dst.copy_(src), 5, 2)
    copy = 2 * src.numel() / (ms * 1e-3) / 1e9
    del src, dst
    a = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda")
    ms = timed_steps(lambda: torch.matmul(a, b), 10, 3)
    gemm = 2 * 8192 ** 3 / (ms * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"copy_GBps": copy, "hbm_spec_GBps": HBM_PEAK_GBPS, "gemm_bf16_TFLOPs": gemm,
            "mfma_bf16_spec_TFLOPs": 2500.0,
            "note": "copy: torch device copy of 4 GiB; gemm: torch.matmul 8192^3 bf16"}


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
    ws = torch.zeros(csa.csa_index_topk_workspace(B, 1, L, HI, k), dtype=torch.uint8, device="cuda")

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
            "note": "scan bound by its per-tile chain (LDS read, MFMA, ReLU and head sum), which two wavefronts per SIMD only partly overlap, not by bytes"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="sequences the CPU oracle decodes (0: one per host core, at most 16 and at most the batch)")
    ap.add_argument("--schedule", choices=SCHEDULES, default="alternate",
                    help="layer schedule of the headline stack (alternate CSA/HCA is the 1M configuration)")
    ap.add_argument("--no-schedules", action="store_true", help="skip the flash / pro schedule measurements")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle step until at least this much oracle time")
    ap.add_argument("--prefill-queries", type=int, default=65536,
                    help="queries of the prefill measurements (the CSA prefill chunk; 0: skip)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the single-layer decode configurations, bulk compression and the measured peaks")
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
    st = Stack(B=args.batch, schedule=args.schedule)
    t_gen = time.perf_counter()
    state = GpuState(st)
    t_gen = time.perf_counter() - t_gen
    print("# inputs generated on the GPU in %.1f s" % t_gen, file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        state.step()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)

    # Timed region: K steps; HIP events bracket one csa_index_topk call (the
    # dominant call) in every fourth step, on the stream it runs on, taking the
    # CSA layers in turn (each bracketed call leaves the GPU idle for a few
    # microseconds around its events, so not every step carries them), and in
    # every step one CSA layer's scan kernel stamps its own start and end.
    ev = {}
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    n_csa = st.kinds().count("csa")
    # in every fourth step (offset by two from the bracketed calls) one CSA
    # layer's scan kernel, the layers in turn, stamps its own start and end
    # (hipExtLaunchKernel events: no command between the kernels, though the
    # stamps still cost the step a few microseconds)
    scan_steps = [i for i in range(args.steps) if i % 4 == 2 or args.steps < 4]
    scan_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in scan_steps]
    for a_, b_ in scan_evs:  # create the events before the timed region
        a_.record()
        b_.record()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        sev = None
        if n_csa and i in scan_steps:
            j = scan_steps.index(i)
            sev = (j % n_csa, scan_evs[j])
        if i % 4 == 0 or args.steps < 4:
            state.step(ev, only=("index_topk",), csa_layer=(i // 4) % n_csa, scan_ev=sev)
        else:
            state.step(scan_ev=sev)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(stop) / args.steps
    idx_ms = event_means_ms(ev)["index_topk"] if ev else None
    scan_ms = sum(a_.elapsed_time(b_) for a_, b_ in scan_evs) / len(scan_evs) if n_csa and scan_evs else None
    print("# timed %d steps: %.3f ms/step (wall %.3f ms/step)" % (args.steps, ms_step, 1e3 * wall / args.steps),
          file=sys.stderr, flush=True)
    # Untimed pass of K steps, each step bracketed by its own events: the
    # median step time (the timed region above gives the mean).
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record()
    for i in range(args.steps):
        state.step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    ms_median = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (step_ms[len(step_ms) // 2 - 1] +
                                                                             step_ms[len(step_ms) // 2])
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
    # the scan kernel alone: the visible keys, the query blocks and head weights
    scan_bytes = (st.nv_csa * st.dI * st.ieb + st.HI * st.dI * st.ieb + st.HI * 4) * st.B
    scan_gbps = scan_bytes / (scan_ms * 1e-3) / 1e9
    scan_traffic = counter_traffic(INDEX_TOPK_SOURCES, st.B, key="index_score_stream_hbm_bytes_per_launch")

    del state
    torch.cuda.empty_cache()
    fp8 = None
    if not args.no_fp8:
        fp8 = fp8_storage_step(args.batch, args.steps, args.warmup)
        print("# fp8 storage: %.3f ms/step" % fp8["ms_per_step"], file=sys.stderr, flush=True)
        fp8["index_topk_mxfp4"] = index_topk_mxfp4(args.batch)
        fp8["fp8_kv_mxfp4_index_step"] = fp8_storage_step(args.batch, args.steps, args.warmup, index_fmt="mxfp4")
        print("# fp8 K/V + mxfp4 indexer: %.3f ms/step" % fp8["fp8_kv_mxfp4_index_step"]["ms_per_step"],
              file=sys.stderr, flush=True)
        print("# mxfp4 index_topk: %.3f ms/call" % fp8["index_topk_mxfp4"]["ms_per_call"], file=sys.stderr,
              flush=True)

    b1 = None
    if args.batch != 1 and not args.no_batch1:
        b1 = decode_step_b1(args.steps, args.warmup, args.schedule)
        print("# batch 1: %.3f ms/step eager, %.3f as a graph" % (b1["ms_per_step"], b1["graph_ms_per_step"]),
              file=sys.stderr, flush=True)
    sched = None
    if not args.no_schedules:
        sched = schedules_b16(args.steps, args.warmup, args.batch)
        print("# schedules: " + ", ".join("%s %.3f ms/step" % (k, v["ms_per_step"]) for k, v in sched.items()),
              file=sys.stderr, flush=True)

    prefill = None
    if args.prefill_queries > 0:
        prefill = prefill_sparse_attn(args.prefill_queries)
        prefill["index_topk"] = prefill_index_topk(args.prefill_queries)
        if not args.no_fp8:
            prefill["index_topk_fp8"] = prefill_index_topk(args.prefill_queries, fp8=True)
            prefill["index_topk_mxfp4"] = prefill_index_topk(args.prefill_queries, mxfp4=True)
            for key, name in (("index_topk_fp8", "E4M3"), ("index_topk_mxfp4", "MXFP4")):
                print("# prefill index + top-k, %s q and keys: %.2f ms (%.0f TFLOP/s)"
                      % (name, prefill[key]["ms_per_call"], prefill[key]["tflops"]), file=sys.stderr, flush=True)
        print("# prefill index + top-k: %.2f ms (%.0f TFLOP/s)" % (prefill["index_topk"]["ms_per_call"],
              prefill["index_topk"]["tflops"]), file=sys.stderr, flush=True)
        print("# prefill sparse attention: %.2f ms for %d queries (%.0f TFLOP/s)"
              % (prefill["ms_per_call"], prefill["queries"], prefill["tflops"]), file=sys.stderr, flush=True)

    configs = None
    if not args.no_configs:
        configs = {"csa_decode_128k_b8": single_layer_decode(args.steps, args.warmup, "csa", 8, 131072, 128),
                   "hca_decode_1m_b4": single_layer_decode(args.steps, args.warmup, "hca", 4, 1_000_000, 0)}
        print("# config 2: %.4f ms/step; config 3: %.4f ms/step" % (configs["csa_decode_128k_b8"]["ms_per_step"],
              configs["hca_decode_1m_b4"]["ms_per_step"]), file=sys.stderr, flush=True)
        configs["csa_compress_bulk_128k_b8"] = bulk_compress("csa", 8, 131072)
        configs["hca_compress_bulk_1m_b4"] = bulk_compress("hca", 4, 1_000_000)
        print("# bulk compress: csa %.0f GB/s, hca %.0f GB/s" % (configs["csa_compress_bulk_128k_b8"]["GBps"],
              configs["hca_compress_bulk_1m_b4"]["GBps"]), file=sys.stderr, flush=True)
        configs["paged_varlen_b16"] = paged_layout(args.batch)
        pl = configs["paged_varlen_b16"]
        print("# paged: index_topk %.3f vs %.3f ms dense, attention %.4f vs %.4f ms dense (identical %s/%s)"
              % (pl["index_topk"]["paged_ms"], pl["index_topk"]["dense_ms"], pl["csa_sparse_attn"]["paged_ms"],
                 pl["csa_sparse_attn"]["dense_ms"], pl["index_topk"]["identical"], pl["csa_sparse_attn"]["identical"]),
              file=sys.stderr, flush=True)
        configs["measured_peaks"] = measured_peaks()
        print("# copy %.0f GB/s, bf16 gemm %.0f TFLOP/s" % (configs["measured_peaks"]["copy_GBps"],
              configs["measured_peaks"]["gemm_bf16_TFLOPs"]), file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        sample = args.cpu_sample or min(16, host_cores(), st.B)
        cpu = cpu_baseline(st, sample, args.cpu_seconds)

    line = {
        "metric": "CSA/HCA decode queries/s at 1M ctx + achieved HBM GB/s (% peak)",
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": ms_median,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(dim) tensors, compressed caches generated in HBM)",
        "config": {
            "workload": "csa_hca_stack8_decode_1M",
            "query": "one token of one sequence through all 8 layers",
            "batch": st.B, "n_ctx": st.n_ctx, "schedule": st.schedule, "layers": ",".join(st.kinds()),
            "heads": st.H, "head_dim": st.d, "index_heads": st.HI, "index_dim": st.dI, "top_k": st.k,
            "window": st.W, "csa_entries": st.L_csa, "hca_entries": st.L_hca,
        },
        "hbm": {"algorithmic_bytes_per_step": st.step_bytes(), "achieved_GBps": step_gbps,
                "frac_of_peak": step_gbps / HBM_PEAK_GBPS},
        "roofline": {"kernel": "index_score_stream<4,true,true,0> (the scan of csa_index_topk, with its part "
                               "selection)",
                     "bound": "hbm", "achieved": scan_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": scan_gbps / HBM_PEAK_GBPS,
                     "traffic": scan_traffic, "avg_launch_ms": scan_ms,
                     "algorithmic_bytes_per_launch": scan_bytes,
                     "timing": "the kernel's own start and end (hipExtLaunchKernel events), one CSA layer in every "
                               "fourth step, the layers in turn, over the timed region",
                     "call": {"kernels": "index_score_stream<4,true,true,0> then topk_merge_kernel",
                              "avg_ms": idx_ms, "algorithmic_bytes": idx_bytes, "achieved": idx_gbps,
                              "frac": idx_gbps / HBM_PEAK_GBPS, "traffic": traffic,
                              "timing": "HIP events around the call in every fourth step (a few us of idle "
                                        "GPU at each event)"}},
        "per_call_ms": per_call,
        "per_call_note": "untimed pass with events around every call; compression runs on a second stream",
        "prefill_sparse_attn": prefill,
        "fp8_storage": fp8,
        "decode_batch1": b1,
        "schedules": sched,
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
