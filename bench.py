"""Benchmark of the QSA layer on one MI355X.

Headline: QSA prefill tokens/s of one layer at 131,072 tokens (B=1,
N(0,1) bf16 inputs with 64 planted needle blocks per KV head, budget 512
blocks).  One step = the whole prefill hot path: RoPE on Q and K, key
pooling, indexer scores + top-K selection, sparse attention.  The same JSON
line also carries the decode step (32 sequences x 262,144 cached tokens),
the same metric at 1M context (an 8,192-query prefill chunk at the end of a
1,048,576-token context, and decode of 4 such sequences), the dense-attention
baselines on the same inputs (speedups), the roofline of the dominant kernel
(HIP events around each launch, on the launch stream), and the fp64 oracle
timed on a bounded sample on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ...]
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

METRIC = "QSA prefill & decode tokens/s at 128K/1M ctx, % roofline, speedup vs dense"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
COPY_BYTES = 1 << 30  # the plain copy that calibrates the HBM byte counters
# HBM counters of the dominant kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE) with
# the hash of the sources they were taken from
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_prefill_128k_hbm_traffic.txt")
# (the kernel's own file, and the types and device helpers of the internal
# header: the text before its launcher declarations)
KERNEL_SOURCES = [os.path.join(ROOT, "block_sparse_long_08_amd", "csrc", f)
                  for f in ("attention.hip", "qsa_internal.h")]
HEADER_CUT = "launchers --"

WORKLOADS = {
    # name: (Tq, pos0, budget, needles per KV head)
    "prefill_2k": (2048, 0, 64, 0),
    "prefill_32k": (32768, 0, 512, 0),
    "prefill_128k": (131072, 0, 512, 64),
    "prefill_1m_chunk": (8192, 1048576 - 8192, 512, 64),
    # the report's prefill condition: 16K-token chunks over a paged cache
    "prefill_1m_chunk16k": (16384, 1048576 - 16384, 512, 64),
}
DECODES = {
    "decode_256k_b32": (32, 262144, 512, 0),
    "decode_1m_b4": (4, 1048576, 512, 64),
}
# speculative decode with index reuse timed on the same caches (the pages'
# decode condition: batch 4, next_n = 4)
DECODE_NEXT_N = {"decode_1m_b4": 4}
# paged-cache variant timed on the same caches (page size in tokens)
DECODE_PAGED = {"decode_1m_b4": 64}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gen_prefill(name, seed=0):
    import synth
    Tq, pos0, budget, nd = WORKLOADS[name]
    t = time.time()
    x = synth.prefill_inputs(Tq, pos0=pos0, seed=seed, needles_per_head=nd,
                             k_is_rotated=pos0 > 0)
    log(f"generated {name} inputs in {time.time() - t:.1f}s")
    return x


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


class StageTimer:
    """HIP events recorded on the launch stream between the stages of a step."""

    def __init__(self, names):
        import torch
        self.names = names
        self.ev = []
        self.torch = torch

    def start_step(self):
        self.cur = [self.torch.cuda.Event(enable_timing=True)]
        self.cur[0].record()

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.cur.append(e)

    def end_step(self):
        self.ev.append(self.cur)

    def per_stage_ms(self):
        out = {n: [] for n in self.names}
        for evs in self.ev:
            for i, n in enumerate(self.names):
                out[n].append(evs[i].elapsed_time(evs[i + 1]))
        return {n: float(np.mean(v)) for n, v in out.items()}


def page_pool(cache, P, perm):
    """Contiguous per-sequence rows [B, L, ...] -> a page pool whose page
    perm[b * (L / P) + i] holds rows i*P .. of sequence b (device copy)."""
    import torch
    B, L = cache.shape[:2]
    rows = cache.reshape(B * (L // P), -1)
    pool = torch.empty_like(rows)
    pool.index_copy_(0, perm, rows)
    return pool.view((B * L,) + tuple(cache.shape[2:]))


def page_table(B, L, P, seed):
    """A random assignment of the B * L / P pages of B sequences to a pool:
    (table [B, L/P] int32 on the device, the permutation as int64 indices)."""
    import torch
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(B * (L // P), generator=g)
    return perm.view(B, L // P).to(torch.int32).cuda(), perm.cuda()


def probe_lib():
    """The gather-ceiling probe (libqsa_probe.so, a measurement kernel built
    beside the layer's library), or None when it is not built."""
    import ctypes
    path = os.path.join(ROOT, "block_sparse_long_08_amd", "libqsa_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.qsa_probe_gather.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, vp, vp]
    lib.qsa_probe_gather.restype = i32
    return lib


# waves per SIMD of the sparse prefill attention (its register cap)
ATTN_WAVES_PER_SIMD = 3


def gather_ceiling(layer, Kr, V, reps):
    """Time the probe over the layer's selection in the attention's row
    launches, each alone on one stream: the time the memory system needs for
    exactly the attention's loads without their arithmetic, at the
    attention's waves per SIMD and at the most the probe can run.
    Returns {waves per SIMD (0 = unrestricted): ms per step}."""
    import torch
    lib = probe_lib()
    if lib is None or layer.pages is not None:
        return None
    out = torch.empty((layer.Tq, layer.Hkv), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for wps in (ATTN_WAVES_PER_SIMD, 0):
        def run():
            for r0, n in layer.attn_chunks():
                st = lib.qsa_probe_gather(Kr.data_ptr(), V.data_ptr(),
                                          layer.blk_idx[r0:].data_ptr(),
                                          layer.n_sel[r0:].data_ptr(), n, layer.pos0 + r0,
                                          layer.budget, layer.Hkv, wps, out[r0:].data_ptr(),
                                          stream)
                if st != 0:
                    raise RuntimeError("qsa_probe_gather rejected its arguments")
        run()
        torch.cuda.synchronize()
        res[wps] = _time_steps(run, reps)
    return res


def bench_prefill(name, steps, warmup, with_dense=True, idx_rope_dim=0, x=None, page_tokens=0,
                  with_distill=False, pipeline_rows=0, with_probe=False, attn_rows=None,
                  kl_rows=None):
    import torch
    import block_sparse_long_08_amd as qsa
    Tq, pos0, budget, nd = WORKLOADS[name]
    x = gen_prefill(name) if x is None else x
    fresh = pos0 == 0
    Q, K, V, qi, ki = map(to_dev, (x.Q, x.K, x.V, x.qi, x.ki))
    Tk = pos0 + Tq
    kbar = None
    pages = None
    if page_tokens:
        # the cache in randomly permuted pages (setup, untimed)
        assert not fresh and Tk % page_tokens == 0
        table, perm = page_table(1, Tk, page_tokens, seed=1)
        pages = qsa.Pages(table, page_tokens)
        K = page_pool(K.view(1, Tk, 2, 256), page_tokens, perm)
        V = page_pool(V.view(1, Tk, 2, 256), page_tokens, perm)
        kbar = torch.empty((Tk // 4, 128), dtype=torch.bfloat16, device="cuda")
        qsa.qsa_compress_keys(ki, 1, pos0, pos0 * 128, 128, 4, 0, kbar, 0,
                              rope_dim=idx_rope_dim, pages=pages)
    elif not fresh:
        # cache of pooled keys for the context before the chunk (setup, untimed)
        kbar = torch.empty((Tk // 4, 128), dtype=torch.bfloat16, device="cuda")
        qsa.qsa_compress_keys(ki, 1, pos0, pos0 * 128, 128, 4, 0, kbar, (pos0 // 4) * 128,
                              rope_dim=idx_rope_dim)
    extra = {} if attn_rows is None else dict(attn_rows=attn_rows)
    if kl_rows is not None:
        extra["kl_rows"] = kl_rows
    layer = qsa.QSAPrefill(Tq, pos0=pos0, budget=budget, fresh=fresh, idx_rope_dim=idx_rope_dim,
                           pages=pages, pipeline_rows=pipeline_rows, **extra)
    torch.cuda.synchronize()
    # the layer's product path: selection and attention overlapped on two
    # streams in row chunks (pipeline_rows), else one after the other
    pipe = layer.pipeline_rows > 0
    names = ["rope_pool", "select_attend"] if pipe else ["rope_pool", "select", "attend"]
    timer = StageTimer(names)
    att_ev, sel_ev = [], []

    def step(t=None):
        if t:
            t.start_step()
        Kr, kb = layer.rope_and_pool(Q, K, ki, kbar)
        qs = layer.rope_indexer(qi)
        if t:
            t.mark()
        if pipe:
            layer.select_and_attend(qs, kb, Kr, V, attn_events=att_ev if t else None,
                                    select_events=sel_ev if t else None)
        else:
            layer.select(qs, kb)
            if t:
                t.mark()
            layer.attend(Kr, V)
        if t:
            t.mark()
            t.end_step()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    stage = timer.per_stage_ms()
    nlaunch = len(layer.attn_chunks())
    if pipe:
        # stage durations from events around each chunk's selection (launch
        # stream) and each attention launch (its own stream); the two overlap,
        # so each is its time beside the other, not its cost alone
        nlaunch = len(att_ev) // steps
        sel_ms = sum(a.elapsed_time(b) for a, b in sel_ev) / steps
        att_ms = sum(a.elapsed_time(b) for a, b in att_ev) / steps
        stage = dict(rope_pool=stage["rope_pool"], select_overlapped=sel_ms,
                     attend_overlapped=att_ms, select_attend=stage["select_attend"])
    # each stage alone on one stream (after the timed steps): every row
    # chunk's selection, then every chunk's attention
    Kr0, kb0 = layer.rope_and_pool(Q, K, ki, kbar)
    qs0 = layer.rope_indexer(qi)
    torch.cuda.synchronize()
    reps = max(1, min(steps, 3))
    stage["select_standalone"] = _time_steps(lambda: layer.select(qs0, kb0), reps)
    stage["attend_standalone"] = _time_steps(lambda: layer.attend_chunks(Kr0, V), reps)
    probe_ms = gather_ceiling(layer, Kr0, V, reps) if with_probe else None
    torch.cuda.synchronize()
    # the outputs of the step's rows for the CPU leg's parity check: the first
    # and last row of every attention launch, rows 0-3 (every (p+1) mod 4
    # trailing-block length) and 64 seeded random rows
    edges = {0, 1, 2, 3, Tq - 1}
    for r0, n in layer.attn_chunks():
        edges |= {r0, r0 + n - 1}
    rs = np.random.default_rng(5).choice(Tq, size=min(64, Tq), replace=False)
    prow = np.array(sorted(edges | set(int(r) for r in rs)), dtype=np.int64)
    pidx = torch.from_numpy(prow).to("cuda")
    res_parity = dict(rows=prow, O=layer.O[pidx].cpu().numpy(), lse=layer.lse[pidx].cpu().numpy(),
                      sel=layer.blk_idx[pidx].cpu().numpy(),
                      nsel=layer.n_sel[pidx].cpu().numpy())
    res = dict(ms_per_step=wall * 1e3, stages_ms=stage, Tq=Tq, Tk=Tk, budget=budget,
               attn_launches=nlaunch, pipeline_rows=layer.pipeline_rows,
               attn_rows=layer.attn_rows, q_rope_on_load=layer.rope_on_load)
    res["attend_launch_ms"] = (att_ms if pipe else stage["attend"]) / nlaunch
    res["_parity"] = res_parity
    if probe_ms is not None:
        res["gather_probe_ms"] = probe_ms
    # algorithmic work of the step
    nsel = layer.n_sel.cpu().numpy().astype(np.int64)
    pos = pos0 + np.arange(Tq)
    ntok = 4 * nsel + (pos + 1) % 4
    gather_bytes = int(ntok.sum()) * 2 * 256 * 2 * 2          # K and V, 2 KV heads, bf16
    attn_bytes = gather_bytes + Tq * 24 * 256 * (2 + 4)        # + Q read, O write (fp32)
    attn_flop = int(ntok.sum()) * 24 * 256 * 2 * 2             # QK^T and PV over 24 heads
    nc = np.minimum((pos + 1) // 4, Tk // 4)
    idx_flop = int(nc.sum()) * 4 * 128 * 2
    res.update(gather_bytes=gather_bytes, attn_bytes=attn_bytes, attn_flop=attn_flop,
               idx_flop=idx_flop, candidates=int(nc.sum()))
    res["dense_flop"] = float(((pos + 1).astype(np.float64)).sum()) * 24 * 256 * 2 * 2
    if with_dense:
        Od = torch.empty((Tq, 24, 256), dtype=torch.float32, device="cuda")
        lse = torch.empty((Tq, 24), dtype=torch.float32, device="cuda")
        Kr = layer.Kr if fresh else K
        dense = lambda: qsa.dense_attn(layer.Qr, Kr, V, 1, Tq, Tk, pos0, None, 24, 2, 256, Od,  # noqa
                                       lse, pages=pages)
        dense()
        torch.cuda.synchronize()
        dsteps = max(1, min(steps, 3))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(dsteps):
            dense()
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / dsteps
        res.update(dense_ms=dms)
        if with_distill and pages is None:
            # stage-1 distillation forward: KL of the indexer against the
            # block-max-pooled dense attention (lse of the dense pass above)
            del Od
            Kr, kb = layer.rope_and_pool(Q, K, ki, kbar)
            qs = layer.rope_indexer(qi)
            wsb = qsa.qsa_distill_workspace_bytes(Tq, Tk)
            ws = torch.empty((max(wsb, 1),), dtype=torch.uint8, device="cuda")
            kl = torch.empty((Tq,), dtype=torch.float32, device="cuda")
            distill = lambda: qsa.qsa_distill_kl(layer.Qr, Kr, lse, qs, kb, Tq, Tk, pos0, 24, 2,  # noqa
                                                 256, 4, 128, 4, 0, kl, ws, wsb)
            distill()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(dsteps):
                distill()
            e1.record()
            torch.cuda.synchronize()
            kms = e0.elapsed_time(e1) / dsteps
            # algorithmic work: q.k over the complete blocks' tokens, 24 heads
            teacher_flop = float((4 * nc).astype(np.float64).sum()) * 24 * 256 * 2
            res["distill"] = dict(ms=kms, teacher_qk_flop=teacher_flop,
                                  teacher_tflops=teacher_flop / (kms * 1e-3) / 1e12,
                                  mfma_frac=teacher_flop / (kms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                  dense_forward_ms=dms, forward_total_ms=dms + kms,
                                  mean_kl=float(kl.mean().item()))
            del ws
            # second stage: the sparse attention fused with the KL under the
            # sparse pattern, over the selection of the timed steps, in the
            # layer's launches of kl_rows rows
            fused = lambda: layer.attend_with_kl(Kr, V, qs, kb, kl)  # noqa: E731
            fused()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(dsteps):
                fused()
            e1.record()
            torch.cuda.synchronize()
            fms = e0.elapsed_time(e1) / dsteps
            res["sparse_kl"] = dict(ms=fms, launches=len(layer._chunks(layer.kl_rows)),
                                    rows_per_launch=layer.kl_rows,
                                    form="staged" if layer.kl_staged else "one kernel",
                                    attend_standalone_ms=stage["attend_standalone"],
                                    vs_attend=fms / stage["attend_standalone"],
                                    hbm_gbps_algorithmic=attn_bytes / (fms * 1e-3) / 1e9,
                                    hbm_frac_algorithmic=attn_bytes / (fms * 1e-3) / 1e9
                                    / HBM_PEAK_GBS,
                                    mean_kl=float(kl.mean().item()))
            # 64 consecutive rows' selection, for the oracle's timing on the host
            r0 = min(Tq - 64, (3 * Tq) // 4)
            res["_kl_sample"] = dict(r0=r0, sel=layer.blk_idx[r0:r0 + 64].cpu().numpy(),
                                     nsel=layer.n_sel[r0:r0 + 64].cpu().numpy())
            del kl
    del layer
    torch.cuda.empty_cache()
    return res, x


def _time_steps(run, steps):
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _decode_rates(B, L, budget, n, ms, dense_ms=None):
    """Throughput and HBM fraction of a decode step of n queries per sequence:
    the pooled keys, the gathered blocks (one selection per sequence) and the
    tail tokens, q read and O written."""
    nb = L // 4
    tail = L - 4 * ((L - n + 1) // 4)  # tokens after the first query's complete blocks
    bytes_step = B * (nb * 128 * 2 + (4 * budget + tail) * 2 * 256 * 2 * 2 + n * 24 * 256 * (2 + 4))
    res = dict(ms_per_step=ms, B=B, L=L, next_n=n, tokens_per_s=B * n / (ms * 1e-3),
               bytes_per_step=bytes_step, hbm_frac=bytes_step / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9))
    # dense decode reads the whole cache once at best: its time at the HBM peak
    dbytes = B * L * 2 * 256 * 2 * 2
    dense_roof_ms = dbytes / (HBM_PEAK_GBS * 1e9) * 1e3
    res.update(dense_at_hbm_peak_ms=dense_roof_ms, speedup_vs_dense_at_hbm_peak=dense_roof_ms / ms)
    if dense_ms is not None:
        res.update(dense_ms=dense_ms, dense_hbm_frac=dbytes / (dense_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                   speedup_vs_dense=dense_ms / ms)
    return res


def bench_decode(name, steps, warmup, with_dense=True):
    import torch
    import block_sparse_long_08_amd as qsa
    import synth
    B, L, budget, nd = DECODES[name]
    t = time.time()
    Kc = torch.empty((B, L, 2, 256), dtype=torch.int16, device="cuda")
    Vc = torch.empty((B, L, 2, 256), dtype=torch.int16, device="cuda")
    kbar = torch.empty((B, L // 4, 128), dtype=torch.int16, device="cuda")
    qh = np.empty((B, 24, 256), dtype=np.uint16)
    qih = np.empty((B, 4, 128), dtype=np.uint16)
    for b in range(B):
        s = synth.decode_seq(b, L, L, needles_per_head=nd)
        Kc[b].copy_(to_dev(s.K))
        Vc[b].copy_(to_dev(s.V))
        kid = to_dev(s.ki)
        qsa.qsa_compress_keys(kid, 1, L, L * 128, 128, 4, 0, kbar[b], (L // 4) * 128)
        qh[b], qih[b] = s.q, s.qi
        del s
    q, qi = to_dev(qh), to_dev(qih)
    torch.cuda.synchronize()
    log(f"generated {name} caches in {time.time() - t:.1f}s")
    seq_len = torch.full((B,), L, dtype=torch.int64, device="cuda")

    def one(n, qq, qqi, kc=Kc, vc=Vc, kb=kbar, pages=None):
        dec = qsa.QSADecode(B, L, budget=budget, next_n=n, pages=pages)
        for _ in range(warmup):
            dec(qq, qqi, kc, vc, kb, seq_len)
        torch.cuda.synchronize()
        ms = _time_steps(lambda: dec(qq, qqi, kc, vc, kb, seq_len), steps)
        dms = None
        if with_dense:
            Od = torch.empty((B, n, 24, 256), dtype=torch.float32, device="cuda")
            wsb = qsa.dense_attn_workspace_bytes(B, n, L, 24, 2, 256)
            ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
            run = lambda: qsa.dense_attn(dec.qr, kc, vc, B, n, L, 0, seq_len, 24, 2, 256, Od,  # noqa
                                         None, ws, wsb, pages=pages)
            run()
            torch.cuda.synchronize()
            dms = _time_steps(run, steps)
            del Od, ws
        on_load = dec.rope_on_load
        del dec
        return dict(_decode_rates(B, L, budget, n, ms, dms), q_rope_on_load=on_load)

    res = one(1, q, qi)
    n = DECODE_NEXT_N.get(name)
    if n:
        # the n newest queries of every sequence (seeded N(0,1) rows)
        qn = to_dev(synth.normal_bf16(1, (B, n, 24, 256), seed=7))
        qin = to_dev(synth.normal_bf16(4, (B, n, 4, 128), seed=7))
        res[f"next_n_{n}"] = one(n, qn, qin)
    P = DECODE_PAGED.get(name)
    if P:
        # the same caches in randomly permuted pages of P tokens (setup, untimed)
        table, perm = page_table(B, L, P, seed=2)
        pages = qsa.Pages(table, P)
        Kp, Vp = page_pool(Kc, P, perm), page_pool(Vc, P, perm)
        kbp = page_pool(kbar, P // 4, perm)
        paged = dict(page_tokens=P, **one(1, q, qi, Kp, Vp, kbp, pages))
        if n:
            paged[f"next_n_{n}"] = one(n, qn, qin, Kp, Vp, kbp, pages)
        res["paged"] = paged
        del Kp, Vp, kbp
    del Kc, Vc, kbar
    torch.cuda.empty_cache()
    return res


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            data = fh.read()
        if f.endswith(".h"):
            data = data.split(HEADER_CUT.encode())[0]
        h.update(data)
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the attention kernel from the committed counter
    summary: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what
    the same counter reads for a plain copy of COPY_BYTES.  None when the
    summary is missing, was taken on another workload, or the kernel's
    sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    try:
        if kv.get("workload") != workload or kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        cb = float(kv["copy_bytes"])
        f_scale = cb / (float(kv["copy_fetch_kib"]) * 1024.0)
        w_scale = cb / (float(kv["copy_write_kib"]) * 1024.0)
        return (float(kv["kernel_fetch_kib"]) * 1024.0 * f_scale +
                float(kv["kernel_write_kib"]) * 1024.0 * w_scale)
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def calibration_copy():
    """One plain device copy of COPY_BYTES (read COPY_BYTES, write COPY_BYTES);
    run under the byte counters it gives their scale."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# The output bar of the parity tests (bf16 inputs, fp32 accumulation).
PARITY_MAX_ABS = 2e-2
PARITY_REL_L2 = 1e-3


def _errors(got, ref):
    d = np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    return float(np.abs(d).max()) if d.size else 0.0, float(np.linalg.norm(d) / den) if den else 0.0


def parity_record(oracle, name, x, Kr, kb, budget, gpu):
    """The timed step's outputs on the sampled rows (gpu: rows, O, lse, sel,
    nsel) against the oracle: the attention over the GPU's own selection
    (every row), the selection itself (rows whose set equals the oracle's),
    and end to end on those rows.  Errors are max-abs and rel-L2 over the
    checked rows, beside the tests' bar."""
    _, pos0, _, _ = WORKLOADS[name]
    rows = gpu["rows"]
    pos = pos0 + rows
    Qr = oracle.rope(x.Q[rows], pos=pos)
    t = time.time()
    ref = oracle.qsa_rows_at(Qr, Kr, x.V, x.qi[rows], kb, pos, Kbudget=budget)
    Oa, la = oracle.sparse_attn_rows_at(Qr, Kr, x.V, pos, gpu["sel"], gpu["nsel"])
    secs = time.time() - t
    same = np.array([gpu["nsel"][i] == ref["nsel"][i] and
                     np.array_equal(gpu["sel"][i, :gpu["nsel"][i]], ref["sel"][i, :ref["nsel"][i]])
                     for i in range(rows.size)])
    att_o, att_l = _errors(gpu["O"], Oa), _errors(gpu["lse"], la)
    rec = dict(rows=int(rows.size),
               sample="first and last row of every attention launch, rows 0-3, 64 seeded "
                      "random rows",
               bar=dict(max_abs=PARITY_MAX_ABS, rel_l2=PARITY_REL_L2),
               attention_on_gpu_selection=dict(O_max_abs=att_o[0], O_rel_l2=att_o[1],
                                               lse_max_abs=att_l[0], lse_rel_l2=att_l[1]),
               selection_equal_rows=int(same.sum()),
               selection_differing_rows=int((~same).sum()), oracle_seconds=secs)
    if same.any():
        e_o, e_l = _errors(gpu["O"][same], ref["O"][same]), _errors(gpu["lse"][same], ref["lse"][same])
        rec["end_to_end_equal_selection"] = dict(O_max_abs=e_o[0], O_rel_l2=e_o[1],
                                                 lse_max_abs=e_l[0], lse_rel_l2=e_l[1])
    rec["within_bar"] = bool(att_o[0] <= PARITY_MAX_ABS and att_o[1] <= PARITY_REL_L2)
    return rec


def cpu_baseline(name, x, budget, seconds=15.0, kl_sample=None, parity=None):
    """The oracle (fp64, OpenMP over rows) on sampled query rows of the
    workload; with parity (the GPU's outputs on a row sample), also the
    parity of those rows against the oracle."""
    import oracle
    Tq, pos0, _, _ = WORKLOADS[name]
    t = time.time()
    Kr = x.K if x.k_is_rotated else oracle.rope(x.K)
    kb = oracle.compress(x.ki)
    prep = time.time() - t
    rng = np.random.default_rng(0)
    rows_done, t_rows = 0, 0.0
    while t_rows < seconds:
        rows = np.sort(rng.choice(np.arange(Tq // 2, Tq), size=64, replace=False))
        pos = pos0 + rows
        Qr = oracle.rope(x.Q[rows], pos=pos)
        t1 = time.time()
        oracle.qsa_rows_at(Qr, Kr, x.V, x.qi[rows], kb, pos, Kbudget=budget)
        t_rows += time.time() - t1
        rows_done += rows.size
    out = dict(value=rows_done / t_rows, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
               cpu_model=cpu_model(), host_logical_cpus=os.cpu_count(),
               sample=f"{rows_done} query rows drawn from the second half of the {name} "
                      f"workload (full QSA per row: scores over every complete block, "
                      f"top-{budget}, attention over the selected tokens, 24 heads); "
                      f"oracle key pooling/RoPE of K ({prep:.1f}s) not counted",
               qsa_extrapolated_s=Tq / (rows_done / t_rows))
    # dense causal attention of 64 consecutive rows at three quarters of the
    # workload; its cost per row grows with the position, so the whole
    # workload is extrapolated per visible token (labelled as such)
    r0 = min(Tq - 64, (3 * Tq) // 4)
    rows = np.arange(r0, r0 + 64)
    Qr = oracle.rope(x.Q[r0:r0 + 64], pos0=pos0 + r0)
    t1 = time.time()
    oracle.dense_rows(Qr, Kr, x.V, rows - r0, pos0=pos0 + r0)
    td = time.time() - t1
    vis = float((pos0 + rows + 1).sum())
    all_vis = float((pos0 + np.arange(Tq, dtype=np.float64) + 1).sum())
    out["dense"] = dict(rows=64, seconds=td, rows_per_s=64 / td,
                        sample=f"rows {r0}..{r0 + 63} of {name} (dense causal attention, 24 heads)",
                        extrapolated_s=td * all_vis / vis)
    if kl_sample is not None:
        # the two distillation KLs: under the sparse pattern on the GPU's
        # selection of 64 consecutive rows, and the stage-1 (dense) KL of 8
        # rows, extrapolated per visible token (labelled as such)
        k0 = kl_sample["r0"]
        Qk = oracle.rope(x.Q[k0:k0 + 64], pos0=pos0 + k0)
        qik = x.qi[k0:k0 + 64]
        t1 = time.time()
        oracle.sparse_kl_rows(Qk, Kr, qik, kb, np.arange(64), kl_sample["sel"], kl_sample["nsel"],
                              pos0=pos0 + k0)
        ts = time.time() - t1
        out["sparse_kl"] = dict(rows=64, seconds=ts, rows_per_s=64 / ts,
                                sample=f"rows {k0}..{k0 + 63} of {name} on the GPU's selection",
                                extrapolated_s=ts * Tq / 64)
        t1 = time.time()
        oracle.distill_rows(Qk[:8], Kr, qik[:8], kb, np.arange(8), pos0=pos0 + k0)
        tdd = time.time() - t1
        v8 = float((pos0 + k0 + np.arange(8) + 1).sum())
        out["distill"] = dict(rows=8, seconds=tdd, rows_per_s=8 / tdd,
                              sample=f"rows {k0}..{k0 + 7} of {name} (stage-1 KL, dense teacher)",
                              extrapolated_s=tdd * all_vis / v8)
    if parity is not None:
        out["parity"] = parity_record(oracle, name, x, Kr, kb, budget, parity)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_128k", choices=sorted(WORKLOADS))
    ap.add_argument("--decode", default="decode_256k_b32", choices=sorted(DECODES) + ["none"])
    ap.add_argument("--dense", default="all", choices=["all", "decode", "none"],
                    help="which dense-attention baselines to time")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--million", default="on", choices=["on", "off"],
                    help="also time the 1M-context workloads (8,192-query prefill chunk, "
                         "decode of 4 sequences) with their dense baselines")
    ap.add_argument("--indexer-rope", default="on", choices=["on", "off"],
                    help="also time the 32K prefill with partial RoPE on the indexer")
    ap.add_argument("--distill", default="on", choices=["on", "off"],
                    help="also time the stage-1 distillation KL on the prefill workload "
                         "(needs the dense baseline's log-sum-exp)")
    ap.add_argument("--pipeline-rows", type=int, default=0,
                    help="rows per selection chunk whose attention overlaps the next chunk's "
                         "selection on a second stream; 0 (default): the selection of all "
                         "rows, then the attention")
    ap.add_argument("--attn-rows", type=int, default=None,
                    help="rows per sparse-attention launch (default: the layer's)")
    ap.add_argument("--kl-rows", type=int, default=None,
                    help="rows per launch of the attention fused with the KL (default: the layer's)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 1 GiB device copy (scale of the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the QSA path here is single-GPU "
              "(multi-GPU sharding is a design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_long_08_amd as qsa
    qsa.qsa_check_device()
    torch.cuda.init()

    if args.calibrate_copy:
        calibration_copy()
    pre, x = bench_prefill(args.workload, args.steps, args.warmup, with_dense=args.dense == "all",
                           with_distill=args.distill == "on", pipeline_rows=args.pipeline_rows,
                           with_probe=True, attn_rows=args.attn_rows, kl_rows=args.kl_rows)
    log(f"prefill {args.workload}: {pre['ms_per_step']:.2f} ms/step, stages {pre['stages_ms']}")
    st = pre["stages_ms"]
    # the dominant kernel of the step is the sparse attention (attn_launches
    # row chunks per step); its launch duration from the timed region
    nl = pre["attn_launches"]
    launch_s = pre["attend_launch_ms"] * 1e-3
    algo = pre["attn_bytes"] / nl            # gathers (no cache reuse), Q, O per launch
    algo_gbps = algo / launch_s / 1e9
    flop = pre["attn_flop"] / nl
    traffic = measured_traffic(args.workload)
    mfma = dict(flop_per_launch=flop, tflops=flop / launch_s / 1e12,
                frac=flop / launch_s / 1e12 / BF16_PEAK_TFLOPS)
    if traffic:
        # the bound: bytes the memory fabric delivered (L2 misses and writes,
        # counter-measured) over the launch duration; the gathers' algorithmic
        # rate passes the HBM peak because the caches serve part of them
        achieved = traffic / launch_s / 1e9
        basis = "measured fabric bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    else:
        achieved = algo_gbps
        basis = "algorithmic bytes, no cache reuse (no counter summary for these kernel sources)"
        log("roofline: the counter summary in profiles/ does not match these attention sources "
            "(take the counter passes again); frac falls back to the no-reuse gather rate, "
            "which is not a bound")
    roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                frac=achieved / HBM_PEAK_GBS, traffic=traffic, basis=basis,
                kernel="attn_prefill_kernel", launch_ms=launch_s * 1e3, launches_per_step=nl,
                algorithmic_bytes=algo, algorithmic_gbps_no_reuse=algo_gbps,
                algorithmic_frac_no_reuse=algo_gbps / HBM_PEAK_GBS, mfma=mfma)
    if "gather_probe_ms" in pre:
        # the same loads by the probe kernel (no arithmetic), each launch
        # alone, against the attention's launches alone over the same rows:
        # at the attention's waves per SIMD, and unrestricted (more waves)
        att_alone = st["attend_standalone"]
        pm = pre["gather_probe_ms"]
        same, free = pm[ATTN_WAVES_PER_SIMD], pm[0]
        best = min(same, free)
        roof["gather_ceiling"] = dict(
            probe_ms_per_step_same_occupancy=same, probe_ms_per_step_unrestricted=free,
            attend_standalone_ms_per_step=att_alone,
            probe_gather_gbps_no_reuse=pre["gather_bytes"] / (best * 1e-3) / 1e9,
            attention_frac_of_ceiling=best / att_alone)
    out = {
        "metric": METRIC,
        "value": pre["Tq"] / (pre["ms_per_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "Tq": pre["Tq"], "context": pre["Tk"],
                   "budget_blocks": pre["budget"], "block": 4, "heads": "24q/2kv x 256",
                   "indexer": "4q/1k x 128", "score_mode": "maxhead", "kbar_mode": "mean",
                   "pipeline_rows": pre["pipeline_rows"], "attn_rows": pre["attn_rows"]},
        "stages_ms": pre["stages_ms"],
        "roofline": roof,
    }
    if "dense_ms" in pre:
        out["dense_prefill_ms"] = pre["dense_ms"]
        out["prefill_speedup_vs_dense"] = pre["dense_ms"] / pre["ms_per_step"]
        out["dense_prefill_tflops"] = pre["dense_flop"] / (pre["dense_ms"] * 1e-3) / 1e12
    if "sparse_kl" in pre:
        out["sparse_kl"] = dict(workload=args.workload, **pre["sparse_kl"])
        log(f"sparse attention + KL {args.workload}: {pre['sparse_kl']['ms']:.2f} ms "
            f"({pre['sparse_kl']['vs_attend']:.2f}x the attention alone)")
    if "distill" in pre:
        out["distill"] = dict(workload=args.workload, **pre["distill"])
        log(f"distill {args.workload}: {pre['distill']['ms']:.2f} ms "
            f"({pre['distill']['teacher_tflops']:.0f} TFLOP/s on q.k)")
    # dense attention at the bf16 MFMA peak: the speedup no dense kernel could shrink
    dense_roof_ms = pre["dense_flop"] / (BF16_PEAK_TFLOPS * 1e12) * 1e3
    out["dense_prefill_at_mfma_peak_ms"] = dense_roof_ms
    out["prefill_speedup_vs_dense_at_mfma_peak"] = dense_roof_ms / pre["ms_per_step"]
    # the step's MFMA work (indexer contraction and attention products) over
    # its wall time: the composite share of the bf16 peak, low by design since
    # the step is bound by the attention's gathers
    comp = (pre["idx_flop"] + pre["attn_flop"]) / (pre["ms_per_step"] * 1e-3) / 1e12
    out["composite_mfma"] = dict(tflops=comp, frac=comp / BF16_PEAK_TFLOPS,
                                 flop=pre["idx_flop"] + pre["attn_flop"])
    if args.indexer_rope == "on":
        # the indexer with partial RoPE (64 of its 128 dims) on the 32K workload,
        # against the same workload without it
        x32 = gen_prefill("prefill_32k")
        plain, _ = bench_prefill("prefill_32k", args.steps, args.warmup, with_dense=False, x=x32)
        rot, _ = bench_prefill("prefill_32k", args.steps, args.warmup, with_dense=False,
                               idx_rope_dim=64, x=x32)
        out["indexer_rope"] = dict(workload="prefill_32k", idx_rope_dim=64,
                                   ms_per_step=rot["ms_per_step"], stages_ms=rot["stages_ms"],
                                   tokens_per_s=rot["Tq"] / (rot["ms_per_step"] * 1e-3),
                                   without_rope_ms_per_step=plain["ms_per_step"],
                                   without_rope_stages_ms=plain["stages_ms"])
        log(f"prefill_32k with indexer RoPE: {rot['ms_per_step']:.2f} ms/step "
            f"(without: {plain['ms_per_step']:.2f})")
        del x32
    if args.decode != "none":
        dec = bench_decode(args.decode, max(args.steps, 10), args.warmup,
                           with_dense=args.dense != "none")
        out["decode"] = dict(workload=args.decode, **dec)
        log(f"decode {args.decode}: {dec['ms_per_step']:.3f} ms/step")
    if args.million == "on":
        # the same metric at 1M context: prefill chunk and decode (own inputs)
        del x
        m_pre, _ = bench_prefill("prefill_1m_chunk", args.steps, args.warmup,
                                 with_dense=args.dense == "all", pipeline_rows=args.pipeline_rows,
                                 attn_rows=args.attn_rows)
        m = dict(workload="prefill_1m_chunk", ms_per_step=m_pre["ms_per_step"],
                 tokens_per_s=m_pre["Tq"] / (m_pre["ms_per_step"] * 1e-3),
                 stages_ms=m_pre["stages_ms"],
                 attend_gather_gbs_no_reuse=m_pre["attn_bytes"] /
                 (m_pre["attend_launch_ms"] * m_pre["attn_launches"] * 1e-3) / 1e9)
        if "dense_ms" in m_pre:
            m.update(dense_ms=m_pre["dense_ms"],
                     speedup_vs_dense=m_pre["dense_ms"] / m_pre["ms_per_step"])
        m_roof = m_pre["dense_flop"] / (BF16_PEAK_TFLOPS * 1e12) * 1e3
        m.update(dense_at_mfma_peak_ms=m_roof,
                 speedup_vs_dense_at_mfma_peak=m_roof / m_pre["ms_per_step"])
        out["prefill_1m_chunk"] = m
        log(f"prefill prefill_1m_chunk: {m_pre['ms_per_step']:.2f} ms/step")
        # the report's prefill condition: a 16K-token chunk over a paged cache
        c_pre, _ = bench_prefill("prefill_1m_chunk16k", args.steps, args.warmup,
                                 with_dense=args.dense == "all", page_tokens=64,
                                 pipeline_rows=args.pipeline_rows, attn_rows=args.attn_rows)
        c = dict(workload="prefill_1m_chunk16k", page_tokens=64, ms_per_step=c_pre["ms_per_step"],
                 tokens_per_s=c_pre["Tq"] / (c_pre["ms_per_step"] * 1e-3),
                 stages_ms=c_pre["stages_ms"])
        if "dense_ms" in c_pre:
            c.update(dense_ms=c_pre["dense_ms"],
                     speedup_vs_dense=c_pre["dense_ms"] / c_pre["ms_per_step"])
        c_roof = c_pre["dense_flop"] / (BF16_PEAK_TFLOPS * 1e12) * 1e3
        c.update(dense_at_mfma_peak_ms=c_roof,
                 speedup_vs_dense_at_mfma_peak=c_roof / c_pre["ms_per_step"])
        out["prefill_1m_chunk16k_paged"] = c
        log(f"prefill prefill_1m_chunk16k (paged): {c_pre['ms_per_step']:.2f} ms/step")
        m_dec = bench_decode("decode_1m_b4", max(args.steps, 10), args.warmup,
                             with_dense=args.dense != "none")
        out["decode_1m_b4"] = dict(workload="decode_1m_b4", **m_dec)
        log(f"decode decode_1m_b4: {m_dec['ms_per_step']:.3f} ms/step")
        if "next_n_4" in m_dec:
            log(f"decode decode_1m_b4 next_n=4: {m_dec['next_n_4']['ms_per_step']:.3f} ms/step")
        x = None
    # QSA against dense attention on the same GPU: measured, and against a
    # dense kernel at the roofline (MFMA peak for prefill, one read of the
    # cache at the HBM peak for decode), which no faster dense kernel can
    # shrink
    sp = {}
    if "prefill_speedup_vs_dense" in out:
        sp[args.workload] = dict(measured=out["prefill_speedup_vs_dense"],
                                 vs_dense_at_roofline=out["prefill_speedup_vs_dense_at_mfma_peak"])
    for key in ("prefill_1m_chunk", "prefill_1m_chunk16k_paged"):
        if key in out and "speedup_vs_dense" in out[key]:
            sp[key] = dict(measured=out[key]["speedup_vs_dense"],
                           vs_dense_at_roofline=out[key]["speedup_vs_dense_at_mfma_peak"])
    for key in ("decode", "decode_1m_b4"):
        d = out.get(key)
        if not d:
            continue
        for name, rec in ((d["workload"], d), (d["workload"] + "_next_n_4", d.get("next_n_4"))):
            if rec and "speedup_vs_dense" in rec:
                sp[name] = dict(measured=rec["speedup_vs_dense"],
                                vs_dense_at_roofline=rec["speedup_vs_dense_at_hbm_peak"])
    out["speedup_vs_dense"] = sp
    if not args.no_cpu:
        if x is None:
            x = gen_prefill(args.workload)
        out["cpu_baseline"] = cpu_baseline(args.workload, x, pre["budget"], args.cpu_seconds,
                                           kl_sample=pre.get("_kl_sample"),
                                           parity=pre.get("_parity"))
        par = out["cpu_baseline"].get("parity")
        if par:
            a = par["attention_on_gpu_selection"]
            log(f"parity on {par['rows']} rows: O max-abs {a['O_max_abs']:.2e} rel-L2 "
                f"{a['O_rel_l2']:.2e}; selection equal on {par['selection_equal_rows']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
