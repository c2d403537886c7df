"""Benchmark of the HCA / DSA forward path on one MI355X.

The timed step is HCA prefill at 131072 tokens (bf16, 16 heads, head_dim 512,
block 128, window 256): block compression of K and V over the whole sequence
followed by attention.  `value` is tokens per second of that step.  The other
workloads of the path are timed in the same run and reported under
`components`:
  * HCA prefill at 32768 tokens (window 128): compression, attention;
  * HCA decode: 64 sequences x 1 query over 8192 compressed entries + 128 raw;
  * DSA prefill at 65536 tokens: indexer + top-2048, sparse attention, and
    the training backward of the sparse attention over the same selections;
  * DSA decode: 16 sequences x 1 query over 1,048,704 positions;
  * CSA prefill at 65536 tokens (the DSA shapes with K, V and the index keys
    compressed by blocks of 4): compression, indexer + top-2048 over the
    16384 entries, sparse attention;
  * attention-output epilogue at the 32768-token HCA shape: the low-rank
    output gate (latent 2048 -> 16 x 512, sigmoid) and VHA mixing (rank 4);
  * HCA training backward at 32768 tokens: the attention backward (dq, dk,
    dv, dkc, dvc) alone, and the layer backward (attention and compressor:
    dk/dv through both paths, the compressor weight gradients).

Inputs are seeded synthetic draws (the library's own generators) already
resident in HBM when timing starts.  Every call is timed by a pair of HIP
events on the stream the library launches on (torch's current stream), one
pair per call, after the 256 MB Infinity Cache has been flushed by writing a
512 MiB scratch buffer (outside the event pair); figures are medians over the
timed calls unless a key says otherwise.  `roofline` is for the dominant
kernel of the step (prefill attention, bound by the matrix cores at this
size): algorithmic FLOPs per launch divided by its mean launch time.
`cpu_baseline` times the float64 oracle on a bounded sample of the same
workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "prefill512_kernel": "sparse_attention_hca_amd/csrc/attn_prefill512.hip",
    "decode512_kernel": "sparse_attention_hca_amd/csrc/attn_decode512.hip",
    "compress_kernel": "sparse_attention_hca_amd/csrc/compress.hip",
    "index_scores_kernel": "sparse_attention_hca_amd/csrc/dsa_index_topk.hip",
    "sparse_attn256_kernel": "sparse_attention_hca_amd/csrc/dsa_attn256.hip",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    with open(os.path.join(ROOT, KERNEL_SOURCES[kernel]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` in `workload` from the committed
    rocprofv3 PMC summary, if it was taken on the current source of this
    kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[f"{kernel}@{workload}"]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def prefill_work(cfg):
    """(FLOPs, algorithmic bytes) of HCA prefill attention: 4*d FLOPs per visible
    (query head, key) pair; Q, O, K, V each moved once plus the compressed cache."""
    import numpy as np
    t = np.arange(cfg.seqlen, dtype=np.int64)
    lo = np.maximum(0, t - cfg.window + 1)
    keys = int((lo // cfg.block + (t - lo + 1)).sum())
    flops = 4.0 * cfg.head_dim * keys * cfg.h_q * cfg.batch
    e = 2
    q = cfg.batch * cfg.seqlen * cfg.h_q * cfg.head_dim * e
    kv = 2 * cfg.batch * cfg.seqlen * cfg.h_kv * cfg.head_dim * e
    cache = 2 * cfg.batch * cfg.n_blocks * cfg.h_kv * cfg.head_dim * e
    return flops, 2 * q + kv + cache


def compress_bytes(cfg):
    e = 2 if cfg.dtype == "bf16" else 4
    nb = cfg.n_blocks
    return 2 * cfg.batch * (nb * cfg.block + nb) * cfg.h_kv * cfg.head_dim * e + 2 * cfg.h_kv * cfg.block * 4


def decode_work(cfg):
    n_keys = cfg.n_blocks + cfg.window
    e = 2
    kv = 2 * cfg.batch * n_keys * cfg.h_kv * cfg.head_dim * e
    qo = 2 * cfg.batch * cfg.h_q * cfg.head_dim * e
    flops = 4.0 * cfg.head_dim * n_keys * cfg.h_q * cfg.batch
    return flops, kv + qo


def dsa_work(cfg):
    S, k = cfg.seqlen, cfg.topk
    pairs_idx = S * (S + 1) // 2
    idx_flops = pairs_idx * (cfg.h_i * (2 * cfg.d_i + 2))
    sel = sum(min(t + 1, k) for t in range(S))
    attn_flops = 2.0 * (cfg.d_qk + cfg.d_v) * cfg.h_q * sel
    return idx_flops, attn_flops, sel


_FLUSH = {}


def mall_flush(torch):
    """Stream a 512 MiB scratch buffer through the caches so that no input of
    the next call is served from the 256 MB Infinity Cache (or the L2s).  The
    buffer is read, not written: a write leaves dirty lines whose write-back
    would land in the next timed call (the decode call measured 0.246 ms after
    a written flush against 0.193 ms back to back)."""
    buf = _FLUSH.get("buf")
    if buf is None:
        buf = _FLUSH["buf"] = torch.ones(128 << 20, dtype=torch.float32, device="cuda:0")
        _FLUSH["out"] = torch.empty((), dtype=torch.float32, device="cuda:0")
    torch.sum(buf, 0, out=_FLUSH["out"])


class Timer:
    """Per-step durations from HIP events on torch's current stream, the stream
    every library call launches on.  A step is one or more calls; an event is
    recorded before the first and after each, so each call of the step has its
    own duration.  The cache flush (when enabled) runs before the first event."""

    def __init__(self, torch, flush=True):
        self.torch = torch
        self.flush = flush
        self.steps = []

    def __call__(self, *fns):
        t = self.torch
        if self.flush:
            mall_flush(t)
        ev = [t.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
        ev[0].record()
        out = []
        for f, e in zip(fns, ev[1:]):
            out.append(f())
            e.record()
        self.steps.append(ev)
        return out

    def durations(self, i=None):
        """ms per step of call i (None: the whole step)."""
        self.torch.cuda.synchronize()
        if i is None:
            return [ev[0].elapsed_time(ev[-1]) for ev in self.steps]
        return [ev[i].elapsed_time(ev[i + 1]) for ev in self.steps]

    def median_ms(self, i=None):
        d = sorted(self.durations(i))
        n = len(d)
        return 0.5 * (d[(n - 1) // 2] + d[n // 2]) if n else float("nan")

    def mean_ms(self, i=None):
        d = self.durations(i)
        return sum(d) / max(1, len(d))


def bench_prefill(torch, hca, synth, cfg, steps, warmup, keep_heads=()):
    """Time `steps` prefill steps (compression, then attention).  Returns the
    medians and means of both calls and of the step, the wall clock of the
    timed loop (flushes included), and, for `keep_heads`, host copies of those
    heads' inputs for the CPU baseline."""
    import numpy as np
    t0 = time.time()
    inp = synth.make_prefill(cfg)
    kept = None
    if keep_heads:
        h = list(keep_heads)
        kept = {n: synth.bf16_bits_to_f32(inp[n][:, :, h]) for n in ("q", "k", "v")}
        kept["w"] = inp["w"][h]
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    del inp["q"], inp["k"], inp["v"]
    w = torch.from_numpy(inp["w"]).to("cuda:0")
    log(f"[bench] {cfg.name}: inputs ready in {time.time() - t0:.1f}s")
    nb = cfg.n_blocks
    kc = torch.empty((cfg.batch, nb, cfg.h_kv, cfg.head_dim), dtype=torch.bfloat16, device="cuda:0")
    vc = torch.empty_like(kc)
    o = torch.empty_like(q)
    lse = torch.empty((cfg.batch, cfg.h_q, cfg.seqlen), dtype=torch.float32, device="cuda:0")
    f1 = lambda: hca.hca_compress_kv(k, v, w, w, cfg.block, kc=kc, vc=vc)
    f2 = lambda: hca.hca_attn_fwd(q, k, v, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale,
                                  o=o, lse=lse)
    for _ in range(warmup):
        f1()
        f2()
    torch.cuda.synchronize()
    tm = Timer(torch)
    start = time.perf_counter()
    for _ in range(steps):
        tm(f1, f2)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - start) * 1e3 / steps
    res = {"compress_ms": tm.median_ms(0), "attn_ms": tm.median_ms(1), "step_ms": tm.median_ms(),
           "compress_mean_ms": tm.mean_ms(0), "attn_mean_ms": tm.mean_ms(1), "step_mean_ms": tm.mean_ms(),
           "wall_ms_per_step_incl_flush": wall_ms, "kept": kept}
    del q, k, v, o, kc, vc, lse
    torch.cuda.empty_cache()
    return res


def bench_decode(torch, hca, synth, cfg, steps, warmup):
    import numpy as np
    inp = synth.make_decode(cfg)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    q, kc, vc, kw, vw = (dev(inp[n]) for n in ("q", "kc", "vc", "kw", "vw"))
    del inp
    o = torch.empty_like(q)
    lse = torch.empty((cfg.batch, cfg.h_q, 1), dtype=torch.float32, device="cuda:0")
    wsz = hca.hca_attn_fwd_workspace_size(cfg.batch, 1, cfg.h_q, cfg.h_kv, cfg.head_dim, cfg.n_blocks, cfg.window)
    ws = torch.empty(wsz, dtype=torch.uint8, device="cuda:0")
    f = lambda: hca.hca_attn_fwd(q, kw, vw, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale,
                                 q_pos0=cfg.q_pos, kv_pos0=cfg.kv_pos0, o=o, lse=lse, workspace=ws)
    for _ in range(warmup):
        f()
    # per call: events around each call, cache flushed before it (median)
    tm = Timer(torch)
    for _ in range(steps):
        tm(f)
    # decode runs token after token: `steps` back-to-back calls between one
    # pair of events, no flush (the 1.09 GB cache exceeds the Infinity Cache)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        f()
    b.record()
    torch.cuda.synchronize()
    res = {"ms": tm.median_ms(), "ms_mean": tm.mean_ms(), "ms_back_to_back": a.elapsed_time(b) / steps}
    # decode-time cache upkeep: one append per token (ring write), plus the
    # block compression on the token that closes a block.  These calls are
    # tiny, so the event-bracketed time is host-bound (argument marshalling
    # and launch); the kernel-trace profile gives the kernels' own durations.
    k_ring = torch.zeros((cfg.batch, 2 * cfg.window, cfg.h_kv, cfg.head_dim), dtype=q.dtype, device="cuda:0")
    v_ring = torch.zeros_like(k_ring)
    w = torch.full((cfg.h_kv, cfg.block), 1.0 / cfg.block, dtype=torch.float32, device="cuda:0")
    t_close = cfg.block * cfg.n_blocks - 1
    t_open = t_close - 1
    for t, key in ((t_open, "append_call_us"), (t_close, "append_close_call_us")):
        g = lambda: hca.hca_append_kv(kw[:, :1], vw[:, :1], k_ring, v_ring, t, cfg.block, w, w, kc, vc)
        for _ in range(warmup):
            g()
        ta = Timer(torch, flush=False)
        for _ in range(steps):
            ta(g)
        res[key] = ta.median_ms() * 1e3
    del q, kc, vc, kw, vw, o, ws, k_ring, v_ring
    torch.cuda.empty_cache()
    return res


def bench_dsa(torch, hca, synth, cfg, steps, warmup, bwd_steps=0):
    import numpy as np
    t0 = time.time()
    inp = synth.make_dsa(cfg)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    qI, kI, w = (torch.from_numpy(inp[n]).to("cuda:0") for n in ("qI", "kI", "w"))
    del inp
    log(f"[bench] {cfg.name}: inputs ready in {time.time() - t0:.1f}s")
    idx = torch.empty((cfg.batch, cfg.seqlen, cfg.topk), dtype=torch.int32, device="cuda:0")
    ws = torch.empty(hca.dsa_index_topk_workspace_size(cfg.batch, cfg.seqlen, cfg.topk), dtype=torch.uint8,
                     device="cuda:0")
    o = torch.empty_like(q)
    lse = torch.empty((cfg.batch, cfg.h_q, cfg.seqlen), dtype=torch.float32, device="cuda:0")
    fi = lambda: hca.dsa_index_topk(qI, kI, w, cfg.topk, idx=idx, workspace=ws)
    fa = lambda: hca.dsa_sparse_attn_fwd(q, k, v, idx, scale=cfg.scale, o=o, lse=lse)
    for _ in range(warmup):
        fi()
        fa()
    tm = Timer(torch)
    for _ in range(steps):
        tm(fi, fa)
    res = {"index_topk_ms": tm.median_ms(0), "attn_ms": tm.median_ms(1), "attn_mean_ms": tm.mean_ms(1)}
    del qI, kI, w, ws
    if bwd_steps:
        # the training backward of the sparse attention over the same selections
        g = torch.Generator(device="cuda:0")
        g.manual_seed(11)
        dout = torch.randn(q.shape, generator=g, device="cuda:0").to(torch.bfloat16)
        wsb = torch.empty(hca.dsa_sparse_attn_bwd_workspace_size(torch.bfloat16, cfg.batch, cfg.seqlen, cfg.h_q, 1,
                                                                 cfg.d_qk, cfg.d_v, cfg.topk),
                          dtype=torch.uint8, device="cuda:0")
        fb = lambda: hca.dsa_sparse_attn_bwd(q, k, v, idx, o, lse, dout, scale=cfg.scale, workspace=wsb)
        fb()
        tmb = Timer(torch)
        for _ in range(bwd_steps):
            tmb(fb)
        res["bwd_ms"] = tmb.median_ms()
        res["bwd_workspace_gb"] = wsb.numel() / 1e9
        del dout, wsb
    del q, k, v, idx, o
    torch.cuda.empty_cache()
    return res


# DSA decode: one query per sequence over the history length of the HCA decode
# workload (1,048,704 positions), c5's indexer and attention shapes.
DSA_DECODE = dict(batch=16, n_keys=1048704, h_i=4, d_i=64, topk=2048, h_q=64, d=256)


def bench_dsa_decode(torch, hca, steps, warmup):
    c = DSA_DECODE
    B, n = c["batch"], c["n_keys"]
    t0 = time.time()
    g = torch.Generator(device="cuda:0")
    g.manual_seed(5)
    kI = torch.randn((B, n, c["d_i"]), generator=g, device="cuda:0")
    qI = torch.randn((B, 1, c["h_i"], c["d_i"]), generator=g, device="cuda:0")
    w = torch.randn((B, 1, c["h_i"]), generator=g, device="cuda:0")
    k = torch.randn((B, n, 1, c["d"]), generator=g, device="cuda:0").to(torch.bfloat16)
    v = torch.randn((B, n, 1, c["d"]), generator=g, device="cuda:0").to(torch.bfloat16)
    q = torch.randn((B, 1, c["h_q"], c["d"]), generator=g, device="cuda:0").to(torch.bfloat16)
    torch.cuda.synchronize()
    log(f"[bench] dsa decode: inputs ready in {time.time() - t0:.1f}s")
    idx = torch.empty((B, 1, c["topk"]), dtype=torch.int32, device="cuda:0")
    ws = torch.empty(hca.dsa_index_topk_decode_workspace_size(B, n, c["topk"]), dtype=torch.uint8, device="cuda:0")
    o = torch.empty_like(q)
    lse = torch.empty((B, c["h_q"]), dtype=torch.float32, device="cuda:0")
    fi = lambda: hca.dsa_index_topk_decode(qI, kI, w, c["topk"], idx=idx, workspace=ws)
    wsa = torch.empty(max(1, hca.dsa_sparse_attn_decode_workspace_size(B, c["h_q"], c["topk"])), dtype=torch.uint8,
                      device="cuda:0")
    fa = lambda: hca.dsa_sparse_attn_decode(q, k, v, idx, scale=1.0 / 16, o=o, lse=lse, workspace=wsa)
    for _ in range(warmup):
        fi()
        fa()
    tm = Timer(torch)
    for _ in range(steps):
        tm(fi, fa)
    ms_i, ms_a = tm.median_ms(0), tm.median_ms(1)
    # indexer: every index key once, the score row written and read back once
    idx_bytes = B * n * (4 * c["d_i"] + 4 + 4)
    # attention: the selected K and V rows (bf16) plus q and o
    attn_bytes = B * c["topk"] * 2 * 2 * c["d"] + 2 * B * c["h_q"] * 2 * c["d"]
    res = {"index_topk_ms": ms_i, "attn_ms": ms_a, "step_ms": ms_i + ms_a,
           "index_gbs": idx_bytes / ms_i / 1e6, "index_hbm_frac": idx_bytes / ms_i / 1e6 / PEAK_HBM_GBS,
           "attn_gbs": attn_bytes / ms_a / 1e6, "tokens_per_s": B / (ms_i + ms_a) * 1e3}
    del kI, qI, w, k, v, q, idx, ws, o
    torch.cuda.empty_cache()
    return res


def csa_work(cfg):
    """(indexer FLOPs, attention FLOPs, selected pairs) of the CSA step."""
    S, k, blk = cfg.seqlen, cfg.topk, cfg.block
    vis = [(t + 1) // blk for t in range(S)]
    idx_flops = sum(vis) * cfg.h_i * (2 * cfg.d_i + 2)
    sel = sum(min(n, k) for n in vis)
    attn_flops = 2.0 * (cfg.d_qk + cfg.d_v) * cfg.h_q * sel
    return idx_flops, attn_flops, sel


def bench_csa(torch, hca, synth, cfg, steps, warmup):
    import numpy as np
    t0 = time.time()
    inp = synth.make_csa(cfg)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    qI, kI, w = (torch.from_numpy(inp[n]).to("cuda:0") for n in ("qI", "kI", "w"))
    wkv, wi = torch.from_numpy(inp["w_kv"]).to("cuda:0"), torch.from_numpy(inp["w_i"]).to("cuda:0")
    del inp
    log(f"[bench] csa: inputs ready in {time.time() - t0:.1f}s")
    n = cfg.n_entries
    kc = torch.empty((cfg.batch, n, 1, cfg.d_qk), dtype=torch.bfloat16, device="cuda:0")
    vc = torch.empty_like(kc)
    kI4 = kI[:, :, None, :]
    kIc4 = torch.empty((cfg.batch, n, 1, cfg.d_i), dtype=torch.float32, device="cuda:0")
    kIc4_v = torch.empty_like(kIc4)
    kIc = kIc4[:, :, 0]
    idx = torch.empty((cfg.batch, cfg.seqlen, cfg.topk), dtype=torch.int32, device="cuda:0")
    ws = torch.empty(hca.csa_index_topk_workspace_size(cfg.batch, cfg.seqlen, n, cfg.topk), dtype=torch.uint8,
                     device="cuda:0")
    o = torch.empty_like(q)
    lse = torch.empty((cfg.batch, cfg.h_q, cfg.seqlen), dtype=torch.float32, device="cuda:0")
    fc = lambda: (hca.hca_compress_kv(k, v, wkv, wkv, cfg.block, kc=kc, vc=vc),
                  hca.hca_compress_kv(kI4, kI4, wi, wi, cfg.block, kc=kIc4, vc=kIc4_v))
    fi = lambda: hca.csa_index_topk(qI, kIc, w, cfg.topk, cfg.block, idx=idx, workspace=ws)
    fa = lambda: hca.csa_sparse_attn_fwd(q, kc, vc, idx, scale=cfg.scale, o=o, lse=lse)
    for _ in range(warmup):
        fc()
        fi()
        fa()
    tm = Timer(torch)
    for _ in range(steps):
        tm(fc, fi, fa)
    res = {"compress_ms": tm.median_ms(0), "index_topk_ms": tm.median_ms(1), "attn_ms": tm.median_ms(2)}
    del q, k, v, qI, kI, w, kc, vc, kIc4, kIc4_v, idx, ws, o, lse
    torch.cuda.empty_cache()
    return res


EPILOGUE = dict(batch=1, seqlen=32768, h=16, d_v=512, d_c=2048, r=4)


def bench_epilogue(torch, hca, steps, warmup):
    e = EPILOGUE
    B, S, H, dv, dc, r = e["batch"], e["seqlen"], e["h"], e["d_v"], e["d_c"], e["r"]
    g = torch.Generator(device="cuda:0")
    g.manual_seed(7)
    o = torch.randn((B, S, H, dv), generator=g, device="cuda:0").to(torch.bfloat16)
    c = torch.randn((B, S, dc), generator=g, device="cuda:0").to(torch.bfloat16)
    w = (torch.randn((H * dv, dc), generator=g, device="cuda:0") / dc ** 0.5).to(torch.bfloat16)
    u = torch.randn((H, r), generator=g, device="cuda:0") * 0.5
    v = torch.randn((r, H), generator=g, device="cuda:0") * 0.5
    y = torch.empty_like(o)
    f = lambda: hca.attn_output_epilogue(o, c, w, u, v, y=y)
    for _ in range(warmup):
        f()
    tm = Timer(torch)
    for _ in range(steps):
        tm(f)
    ms = tm.median_ms()
    flops = 2.0 * B * S * H * dv * dc
    byts = 2 * (B * S * dc + H * dv * dc + 2 * B * S * H * dv)
    del o, c, w, u, v, y
    torch.cuda.empty_cache()
    return {"ms": ms, "tokens_per_s": B * S / ms * 1e3, "gate_tflops": flops / ms / 1e9,
            "gate_mfma_frac": flops / ms / 1e9 / PEAK_BF16_TFLOPS, "gbs": byts / ms / 1e6,
            "flops": flops, "algorithmic_bytes": byts}


def backward_work(cfg):
    """(FLOPs, algorithmic bytes) of the HCA attention backward: 10*d FLOPs per
    visible (query head, key) pair (S, dP, dQ, dK, dV); reads Q, K, V, O, dO
    (bf16), the compressed cache and the LSE once, writes dQ, dK, dV, dKc, dVc
    (fp32) once."""
    flops, _ = prefill_work(cfg)
    flops *= 10.0 / 4.0
    e = 2
    qo = cfg.batch * cfg.seqlen * cfg.h_q * cfg.head_dim
    kv = cfg.batch * cfg.seqlen * cfg.h_kv * cfg.head_dim
    cache = cfg.batch * cfg.n_blocks * cfg.h_kv * cfg.head_dim
    reads = e * (3 * qo + 2 * kv + 2 * cache) + 4 * cfg.batch * cfg.h_q * cfg.seqlen
    writes = 4 * (qo + 2 * kv + 2 * cache)
    return flops, reads + writes


def bench_backward(torch, hca, synth, cfg, steps, warmup):
    """Forward once (compression + attention), then two timed backward calls:
    hca_attn_bwd alone (attention gradients) and hca_attn_compress_bwd (the
    layer's whole backward: attention and compressor, dk/dv through both
    paths, dw)."""
    import numpy as np
    t0 = time.time()
    inp = synth.make_prefill(cfg)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    del inp["q"], inp["k"], inp["v"]
    w = torch.from_numpy(inp["w"]).to("cuda:0")
    dout = dev(synth.make_normal((cfg.batch, cfg.seqlen, cfg.h_q, cfg.head_dim), cfg.seed + 1, cfg.std, bf16=True))
    log(f"[bench] backward: inputs ready in {time.time() - t0:.1f}s")
    kc, vc = hca.hca_compress_kv(k, v, w, w, cfg.block)
    o, lse = hca.hca_attn_fwd(q, k, v, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale)
    ws = torch.empty(hca.hca_attn_bwd_workspace_size(torch.bfloat16, cfg.batch, cfg.seqlen, 0, cfg.n_blocks, cfg.h_q,
                                                     cfg.h_kv, cfg.head_dim, cfg.block, cfg.window),
                     dtype=torch.uint8, device="cuda:0")
    fa = lambda: hca.hca_attn_bwd(q, k, v, kc, vc, o, lse, dout, window=cfg.window, block=cfg.block,
                                  scale=cfg.scale, workspace=ws)
    fl = lambda: hca.hca_attn_compress_bwd(q, k, v, kc, vc, o, lse, dout, w, w, window=cfg.window,
                                           block=cfg.block, scale=cfg.scale, workspace=ws)
    res = {}
    for name, f in (("attn_bwd_ms", fa), ("layer_bwd_ms", fl)):
        for _ in range(warmup):
            f()
        tm = Timer(torch)
        for _ in range(steps):
            tm(f)
        res[name] = tm.median_ms()
        torch.cuda.empty_cache()
    del q, k, v, o, lse, dout, kc, vc, ws
    torch.cuda.empty_cache()
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, kept, row_stride=4):
    """The float64 oracle, as it stands, on a bounded sample of the headline
    step: for the kept heads, compression of all their blocks (K and V) and attention
    for every `row_stride`-th query row; BLAS held to one thread, so one core
    does all the work.  Scaled to tokens/s of the whole step (all heads, all
    rows; the strided rows cover the whole range of key counts)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    blas = ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info()) or "none"
    heads = kept["q"].shape[2]
    q, k, v = (kept[n].astype(np.float64) for n in ("q", "k", "v"))
    rows = list(range(0, cfg.seqlen, row_stride))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        kc = oracle.compress_kv(k, kept["w"], cfg.block)
        vc = oracle.compress_kv(v, kept["w"], cfg.block)
        t_comp = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.hca_attention(q, k, v, kc, vc, window=cfg.window, block=cfg.block, scale=cfg.scale, rows=rows)
        t_attn = time.perf_counter() - t0
    est = (t_comp + t_attn * cfg.seqlen / len(rows)) * cfg.h_q / heads
    return {"value": cfg.seqlen / est, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"float64 oracle on {heads} of {cfg.h_q} heads of the {cfg.seqlen}-token prefill: "
                      f"compression of every block ({t_comp:.1f}s) and attention for every {row_stride}th "
                      f"query row ({len(rows)} rows, {t_attn:.1f}s), scaled to all rows and heads "
                      f"(estimated {est:.0f}s for the whole step)",
            "cpu_model": _cpu_model(), "blas": blas, "threads": 1}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="c2,c4,c5,c5b,c5d,csa,epi,bwd",
                    help="comma list of component workloads to run besides the headline step (c3 always runs; "
                         "'copy' runs only the counter calibration copy)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
              f"(the path needs no cross-GPU exchange; see the sharding note in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_hca_amd as hca
    import synth
    hca.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    only = set(args.only.split(","))
    if "copy" in only:
        # Calibration leg for the HBM traffic counters: a plain device copy of a
        # known size, profiled with the same counters as the attention kernels.
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                          "launches": 5}), flush=True)
        return
    comps = {}

    c3 = synth.CONFIGS["c3"]
    steps3 = max(20, args.steps)
    r3 = bench_prefill(torch, hca, synth, c3, steps3, max(2, args.warmup),
                       keep_heads=() if args.no_cpu_baseline else (0, 8))
    f3, b3 = prefill_work(c3)
    comps["hca_prefill_128k"] = {
        "compress_ms": r3["compress_ms"], "attn_ms": r3["attn_ms"], "e2e_ms": r3["step_ms"],
        "attn_mean_ms": r3["attn_mean_ms"], "timed_steps": steps3,
        "tokens_per_s": c3.seqlen / r3["step_ms"] * 1e3,
        "attn_tflops": f3 / r3["attn_ms"] / 1e9, "attn_mfma_frac": f3 / r3["attn_ms"] / 1e9 / PEAK_BF16_TFLOPS,
        "attn_gbs": b3 / r3["attn_ms"] / 1e6,
        "compress_gbs": compress_bytes(c3) / r3["compress_ms"] / 1e6,
        "compress_hbm_frac": compress_bytes(c3) / r3["compress_ms"] / 1e6 / PEAK_HBM_GBS,
    }
    log(f"[bench] c3 done: {comps['hca_prefill_128k']}")

    if "c2" in only:
        c2 = synth.CONFIGS["c2"]
        r2 = bench_prefill(torch, hca, synth, c2, max(20, args.steps), args.warmup)
        f2, b2 = prefill_work(c2)
        comps["hca_prefill_32k"] = {
            "compress_ms": r2["compress_ms"], "attn_ms": r2["attn_ms"], "e2e_ms": r2["step_ms"],
            "tokens_per_s": c2.seqlen / r2["step_ms"] * 1e3,
            "attn_tflops": f2 / r2["attn_ms"] / 1e9, "attn_mfma_frac": f2 / r2["attn_ms"] / 1e9 / PEAK_BF16_TFLOPS,
            "attn_gbs": b2 / r2["attn_ms"] / 1e6, "attn_hbm_frac": b2 / r2["attn_ms"] / 1e6 / PEAK_HBM_GBS,
            "attn_traffic_bytes": measured_traffic("prefill512_kernel", "hca_prefill_32k"),
            "compress_gbs": compress_bytes(c2) / r2["compress_ms"] / 1e6,
        }
        log(f"[bench] c2 done: {comps['hca_prefill_32k']}")
    if "c4" in only:
        c4 = synth.CONFIGS["c4"]
        r4 = bench_decode(torch, hca, synth, c4, max(20, args.steps), args.warmup)
        f4, b4 = decode_work(c4)
        comps["hca_decode_1m"] = {
            "ms": r4["ms"], "ms_mean": r4["ms_mean"], "ms_back_to_back": r4["ms_back_to_back"],
            "gbs": b4 / r4["ms"] / 1e6, "hbm_frac": b4 / r4["ms"] / 1e6 / PEAK_HBM_GBS,
            "hbm_frac_back_to_back": b4 / r4["ms_back_to_back"] / 1e6 / PEAK_HBM_GBS,
            "tokens_per_s": c4.batch / r4["ms"] * 1e3, "tflops": f4 / r4["ms"] / 1e9,
            "append_call_us": r4["append_call_us"], "append_close_call_us": r4["append_close_call_us"],
        }
        log(f"[bench] c4 done: {comps['hca_decode_1m']}")
    if "c5" in only:
        c5 = synth.CONFIGS["c5"]
        r5 = bench_dsa(torch, hca, synth, c5, max(5, args.steps // 4), 1, bwd_steps=3 if "c5b" in only else 0)
        fi, fa, sel = dsa_work(c5)
        tot = r5["index_topk_ms"] + r5["attn_ms"]
        comps["dsa_prefill_64k"] = {
            "index_topk_ms": r5["index_topk_ms"], "attn_ms": r5["attn_ms"], "e2e_ms": tot,
            "tokens_per_s": c5.seqlen / tot * 1e3,
            "index_tflops_f32": fi / r5["index_topk_ms"] / 1e9,
            "attn_tflops": fa / r5["attn_ms"] / 1e9, "attn_mfma_frac": fa / r5["attn_ms"] / 1e9 / PEAK_BF16_TFLOPS,
        }
        if "bwd_ms" in r5:
            # per selected (query, position) pair and head: S, dP, dQ, dK, dV (5 x 2 x 256 FLOPs)
            fbw = 2.0 * 5 * c5.d_qk * c5.h_q * sel
            comps["dsa_backward_64k"] = {
                "ms": r5["bwd_ms"], "tokens_per_s": c5.seqlen / r5["bwd_ms"] * 1e3,
                "tflops": fbw / r5["bwd_ms"] / 1e9, "mfma_frac": fbw / r5["bwd_ms"] / 1e9 / PEAK_BF16_TFLOPS,
                "flops": fbw, "workspace_gb": r5["bwd_workspace_gb"],
            }
        log(f"[bench] c5 done: {comps['dsa_prefill_64k']} {comps.get('dsa_backward_64k', '')}")
    if "c5d" in only:
        comps["dsa_decode_1m"] = bench_dsa_decode(torch, hca, max(20, args.steps), args.warmup)
        log(f"[bench] c5d done: {comps['dsa_decode_1m']}")

    if "csa" in only:
        cc = synth.CSA_CONFIGS["csa64k"]
        rc = bench_csa(torch, hca, synth, cc, max(5, args.steps // 4), 1)
        fi_c, fa_c, sel_c = csa_work(cc)
        tot = rc["compress_ms"] + rc["index_topk_ms"] + rc["attn_ms"]
        comps["csa_prefill_64k"] = {
            "compress_ms": rc["compress_ms"], "index_topk_ms": rc["index_topk_ms"], "attn_ms": rc["attn_ms"],
            "e2e_ms": tot, "tokens_per_s": cc.seqlen / tot * 1e3,
            "index_tflops_f32": fi_c / rc["index_topk_ms"] / 1e9,
            "attn_tflops": fa_c / rc["attn_ms"] / 1e9,
            "attn_mfma_frac": fa_c / rc["attn_ms"] / 1e9 / PEAK_BF16_TFLOPS,
        }
        log(f"[bench] csa done: {comps['csa_prefill_64k']}")
    if "epi" in only:
        comps["attn_epilogue_32k"] = bench_epilogue(torch, hca, max(20, args.steps), args.warmup)
        log(f"[bench] epilogue done: {comps['attn_epilogue_32k']}")
    if "bwd" in only:
        c2 = synth.CONFIGS["c2"]
        rb = bench_backward(torch, hca, synth, c2, max(10, args.steps // 2), 2)
        fb, bb = backward_work(c2)
        comps["hca_backward_32k"] = {
            "attn_bwd_ms": rb["attn_bwd_ms"], "layer_bwd_ms": rb["layer_bwd_ms"],
            "layer_bwd_tokens_per_s": c2.seqlen / rb["layer_bwd_ms"] * 1e3,
            "attn_bwd_tflops": fb / rb["attn_bwd_ms"] / 1e9,
            "attn_bwd_mfma_frac": fb / rb["attn_bwd_ms"] / 1e9 / PEAK_BF16_TFLOPS,
            "attn_bwd_gbs": bb / rb["attn_bwd_ms"] / 1e6,
            "attn_bwd_hbm_frac": bb / rb["attn_bwd_ms"] / 1e6 / PEAK_HBM_GBS,
            "algorithmic_bytes": bb, "flops": fb,
        }
        log(f"[bench] bwd done: {comps['hca_backward_32k']}")

    value = c3.seqlen / r3["step_ms"] * 1e3
    achieved = f3 / r3["attn_mean_ms"] / 1e9
    line = {
        "metric": "HCA prefill tokens/s + TFLOP/s (% MFMA peak); decode GB/s (% HBM peak)",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps3, "warmup": max(2, args.warmup),
        "ms_per_step": r3["step_ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "HCA prefill bf16: batch 1, seq 131072, 16 heads, head_dim 512, block 128 "
                               "(1024 compressed entries), window 256; step = hca_compress_kv over the whole "
                               "sequence + hca_attn_fwd",
                   "global_batch": 1, "seq_len": c3.seqlen, "parallelism": "none (1 GPU)",
                   "timing": "median of per-step HIP-event durations, Infinity Cache flushed before each step",
                   "wall_ms_per_step_incl_flush": r3["wall_ms_per_step_incl_flush"]},
        "roofline": {"bound": "mfma", "kernel": "prefill512_kernel", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic("prefill512_kernel", "hca_prefill_128k"),
                     "algorithmic_flops_per_launch": f3, "algorithmic_bytes_per_launch": b3,
                     "launch_ms_mean": r3["attn_mean_ms"], "launch_ms_median": r3["attn_ms"]},
        "components": comps,
    }
    if not args.no_cpu_baseline:
        t0 = time.time()
        line["cpu_baseline"] = cpu_baseline(c3, r3["kept"])
        log(f"[bench] cpu baseline took {time.time() - t0:.1f}s")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
