"""Throughput of the FP8 paged decode step on one MI355X.

A step is one pass of the whole hot path over a batch of decode requests:
the tag check, the append of each request's new token, split-KV decode and
the merge. Grouped-query shapes run it in two launches (pkv_step_decode, the
decode with each split's tag check and the new token read from its values;
pkv_step_combine, the merge with the verdicts and the append); the others in
three (pkv_verify_append -> pkv_decode_attn -> pkv_combine).
Before every timed step a 1 GiB buffer is written and read back
(pkv_fill_u32, pkv_read_u32), which evicts the 256 MB last-level cache as
the model's other layers would between two decode steps of one layer (the
read makes the write-back of the dirty lines happen there, not in the
step); the step's launches are then bracketed by HIP events on its
stream. The flush keeps the GPU busy far longer than the host takes to
issue the launches, so the figure holds no host time.
``ms_per_step`` is the median of those flushed steps (with a distribution-free
95% confidence interval). Beside it: the same step captured once as a HIP
graph and replayed after each flush (a graph launch costs a fixed few
microseconds more on this ROCm), and warm figures (graph replays back to
back, no flush). A separate flushed eager pass times the decode kernel
alone with events on the stream it is launched on (the roofline figure).
Default workload: the concurrency-sweep point at batch 64 (contexts uniform
on [2048, 32768], 64 query / 8 KV heads, head dim 128, page 16, per-head
e4m3 scales, tag check on). Inputs are built on the GPU before timing.

Printed: one JSON line. ``value`` is KV GB/s of the step (e4m3 cache bytes
read by the step / median flushed step time); also sequence-steps/s, the
BF16-cache step for comparison, the decode kernel's roofline (its algorithmic
bytes over its average flushed duration) and the oracle on the host's cores
as a CPU baseline (run first, before the GPU is touched).

    python bench.py [--steps K] [--warmup W] [--batch B] [--no-bf16]
                    [--no-cpu-baseline] [--sweep] [--integrity]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK = 2500.0  # TFLOP/s, dense
FLUSH_BYTES = 1 << 30    # written, then read, before every timed step: 4x the 256 MB MALL

# HBM traffic of the decode kernel from rocprofv3 --pmc runs of this same
# command (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, mean over the
# dispatches), keyed by (workload, split, sha256 prefix of the kernel source
# and every header beside it, as the counters were taken on). A plain 1 GiB device copy reads as 524,300 KiB
# FETCH_SIZE and 1,048,576 KiB WRITE_SIZE, so FETCH_SIZE counts in units of 2 KiB
# here and WRITE_SIZE in KiB. Entries stop matching once the kernel changes.
FETCH_FACTOR, WRITE_FACTOR = 2.0, 1.0
TRAFFIC_KIB = {
    ("sweep_b64", 2048, "decode_gqa_mfma.hip", "fe2d55f8c160c1d2"): (1197492.6, 20029.6),
    ("mla_b64", 256, "decode_mla.hip", "695033e6be803fe4"): (195725.4, 81508.0),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--workload", default="sweep", choices=["sweep", "gqa", "long", "mla"],
                    help="sweep: concurrency-sweep point (--batch); gqa: batch 8 x 4096; "
                         "long: batch 4 x 131072, 256-token splits; mla: wide latent head")
    ap.add_argument("--split", type=int, default=0, help="split tokens (0 = library's suggestion)")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="also time batch 1/8/16/32")
    ap.add_argument("--integrity", action="store_true",
                    help="also time verify on/off at batch 1/2/4/8, context 8692")
    ap.add_argument("--handoff", action="store_true",
                    help="also time pkv_requantize_pages: 8192 BF16 pages (Hkv 8, page 16, "
                         "head dim 128) re-encoded into an e4m3 pool")
    ap.add_argument("--drafts", type=int, default=0, metavar="T",
                    help="also time decode of a token and T-1 drafts per request on the same cache")
    ap.add_argument("--row-scales", action="store_true",
                    help="also time the workload with scales set at append, one per cached row")
    ap.add_argument("--int4", action="store_true",
                    help="also time the INT4 weight-only linear layer at batch 1..64")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def kernel_digest(src: str) -> str:
    """sha256 prefix over a kernel source and the csrc headers (any of which
    the kernel may include), in a fixed order."""
    import glob
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "decode_attention_fp8_amd", "csrc")
    h = hashlib.sha256()
    for path in [os.path.join(d, src)] + sorted(glob.glob(os.path.join(d, "*.h"))):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(w, split: int):
    """Scaled HBM bytes per decode launch, or None if no counters match."""
    src = "decode_mla.hip" if w.latent else "decode_gqa_mfma.hip"
    digest = kernel_digest(src)
    kib = TRAFFIC_KIB.get((w.name, split, src, digest))
    if kib is None:
        return None
    return int(round((kib[0] * FETCH_FACTOR + kib[1] * WRITE_FACTOR) * 1024))


def kv_bytes(w, elem_bytes: int, read=None) -> int:
    """Cache bytes the step reads: every token of every request that is not
    aborted (read: bool [B] from the device's abort flags; None = all)."""
    per_token = w.num_kv_heads * (w.head_dim_k if w.latent else w.head_dim_k + w.head_dim_v)
    lens = w.seq_lens.astype("int64")
    if read is not None:
        lens = lens[read]
    return int(lens.sum()) * per_token * elem_bytes


class Runner:
    """Device state of one workload and its timed step."""

    def __init__(self, w, kv_dtype: str, split: int | None, verify: bool = True,
                 row_scales: bool = False):
        import numpy as np
        import torch

        import decode_attention_fp8_amd as pkv
        self.torch, self.pkv, self.w = torch, pkv, w
        dev = "cuda"
        c = pkv.allocate_cache(w.num_pages, w.num_kv_heads, w.page_size, w.head_dim_k,
                               w.head_dim_v, kv_dtype, w.latent, dev, row_scales=row_scales)
        k = w.k_all(dev)
        v = None if w.latent else w.v_all(dev)
        if kv_dtype == "fp8" and not row_scales:
            pkv.pkv_scales_from_amax(k, w.per_head_scales, c.k_scale)
            if w.latent:
                c.v_scale = c.k_scale
            else:
                pkv.pkv_scales_from_amax(v, w.per_head_scales, c.v_scale)
        slot = torch.from_numpy(w.slots()).to(dev)
        pkv.pkv_append(c, k, v, slot)
        off = w.token_offsets()
        last = torch.from_numpy(off[1:] - 1).to(dev)
        self.new_k = k[last].contiguous()
        self.new_v = None if v is None else v[last].contiguous()
        self.new_slot = slot[last].contiguous()
        del k, v, slot
        self.new_req = torch.arange(w.batch, dtype=torch.int32, device=dev)
        c.page_tags = torch.from_numpy(w.page_tags.view(np.int32).copy()).to(dev)
        self.bt = torch.from_numpy(w.block_table).to(dev)
        self.exp = torch.from_numpy(w.expected_tags.view(np.int32).copy()).to(dev)
        self.lens = torch.from_numpy(w.seq_lens).to(dev)
        self.q = w.q_values(dev)
        self.cache = c
        self.step = pkv.DecodeStep(c, w.num_q_heads, w.batch, int(w.seq_lens.max()),
                                   split or w.split_tokens, verify, dev,
                                   total_tokens=w.total_tokens)
        # each request's new token sits at its last position, so the shapes
        # that have it take the two-launch step
        self.two_launch = pkv.pkv_step_launches(c, w.num_q_heads, self.step.split_tokens) == 2
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    def one(self, ev=None):
        pkv, s = self.pkv, self.step
        abort = None
        if self.two_launch:
            # the whole step in two launches: the tag check inside the decode
            # launch, the append inside the merge
            if ev is not None:
                ev[0].record()
            exp = self.exp if s.verify else None  # None: the step without the check
            pkv.pkv_step_decode(self.cache, self.q, self.new_k, self.new_v, self.bt, exp,
                                self.lens, s.max_seq_len, self.w.sm_scale, s.split_tokens,
                                s.o_part, s.lse_part, s.unit_flags, s.abort)
            if ev is not None:
                ev[1].record()
            pkv.pkv_step_combine(self.cache, self.new_k, self.new_v, self.bt, exp, self.lens,
                                 s.max_seq_len, s.split_tokens, s.o_part, s.lse_part,
                                 s.unit_flags, s.abort, s.out, s.lse)
            return
        if s.verify:
            # the check and the append of each request's new token, one launch
            pkv.pkv_verify_append(self.cache, self.bt, self.exp, self.lens, s.abort, self.new_k,
                                  self.new_v, self.new_slot)
            abort = s.abort
        else:
            pkv.pkv_append(self.cache, self.new_k, self.new_v, self.new_slot)
        if ev is not None:
            ev[0].record()
        pkv.pkv_decode_attn(self.cache, self.q, self.bt, self.lens, s.max_seq_len, abort,
                            self.w.sm_scale, s.split_tokens, s.o_part, s.lse_part)
        if ev is not None:
            ev[1].record()
        pkv.pkv_combine(s.o_part, s.lse_part, self.lens, s.split_tokens, s.max_seq_len, abort,
                        s.out, s.lse)

    def capture(self):
        """The whole step as one HIP graph (the step's launches only)."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.one()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.one()
        torch.cuda.synchronize()
        return g

    def time(self, steps: int, warmup: int, flush=None) -> dict:
        """Flushed and warm timings of the step (milliseconds).

        decode: a flushed eager pass, each step's decode launch bracketed by
          events on its stream (the kernel's own duration).
        flushed: the step's launches issued after each flush and
          bracketed by events. The flush keeps the GPU busy for far longer
          than the host takes to issue them, so no host time is in the
          figure (were the host late, the gap would count against it).
        flushed_graph: the captured step replayed once per flush (a graph
          launch adds a fixed cost on this ROCm, reported for comparison).
        warm: replays back to back without a flush; the graph keeps the host
          from bounding small steps. Each list holds one time per step; the
          headline is the flushed median."""
        torch = self.torch
        flush = flush or Flusher()
        ev = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for _ in range(warmup):
            flush()
            self.one()
        evs = [ev() for _ in range(steps)]
        torch.cuda.synchronize()
        for e in evs:
            flush()
            self.one(e)
        torch.cuda.synchronize()
        dec = [a.elapsed_time(b) for a, b in evs]
        fl = [ev() for _ in range(steps)]
        t0 = time.perf_counter()
        for a, b in fl:
            flush()
            a.record()
            self.one()
            b.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        g = self.capture()
        for _ in range(warmup):
            flush()
            g.replay()
        fg = [ev() for _ in range(steps)]
        torch.cuda.synchronize()
        for a, b in fg:
            flush()
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        wm = [ev() for _ in range(steps)]
        for a, b in wm:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        del g
        return {"flushed": [a.elapsed_time(b) for a, b in fl],
                "flushed_graph": [a.elapsed_time(b) for a, b in fg],
                "warm": [a.elapsed_time(b) for a, b in wm],
                "decode": dec,
                "wall_ms_per_flushed_step": (t1 - t0) * 1e3 / steps}


class Flusher:
    """Evicts the last-level cache on the current stream: writes FLUSH_BYTES
    with the library's fill kernel (a new value each call), then reads them
    back with its read kernel, so that the dirty lines the writes leave are
    written back here and not inside the next timed step."""

    def __init__(self):
        import torch

        import decode_attention_fp8_amd as pkv
        self.pkv = pkv
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.n = 0

    def __call__(self):
        self.n += 1
        self.pkv.pkv_fill_u32(self.buf, self.n)
        self.pkv.pkv_read_u32(self.buf, self.sink)


def median_ci(xs):
    """(median, lo, hi): the sample median and a distribution-free 95%
    confidence interval for the median, between the order statistics j and
    n + 1 - j with j the 2.5% quantile of Binomial(n, 1/2)."""
    from scipy.stats import binom
    v = sorted(xs)
    n = len(v)
    med = (v[(n - 1) // 2] + v[n // 2]) / 2
    j = int(binom.ppf(0.025, n, 0.5))
    if j < 1:
        return med, v[0], v[-1]
    return med, v[j - 1], v[n - j]


def summary(t: dict) -> dict:
    """Median, 95% CI and mean of the flushed, graph, warm and decode timings."""
    out = {}
    for key in ("flushed", "flushed_graph", "warm", "decode"):
        med, lo, hi = median_ci(t[key])
        out[key] = {"median_ms": round(med, 5), "ci95_ms": [round(lo, 5), round(hi, 5)],
                    "mean_ms": round(sum(t[key]) / len(t[key]), 5)}
    out["wall_ms_per_flushed_step"] = round(t["wall_ms_per_flushed_step"], 5)
    return out


def time_handoff(steps: int, n_pages: int = 8192):
    """pkv_requantize_pages over n_pages BF16 pages (Hkv 8, page 16, head dim
    128; seeded N(0,1) values) into an e4m3 pool, pages in a random order.
    Bytes moved: 2 B read + 1 B written per value, K and V."""
    import torch

    import decode_attention_fp8_amd as pkv
    H, P, D = 8, 16, 128
    g = torch.Generator(device="cuda").manual_seed(1007)
    src = pkv.allocate_cache(n_pages, H, P, D, D, "bf16", False, "cuda", poison=False)
    src.k_pool.copy_(torch.randn(src.k_pool.shape, generator=g, device="cuda"))
    src.v_pool.copy_(torch.randn(src.v_pool.shape, generator=g, device="cuda"))
    dst = pkv.allocate_cache(n_pages, H, P, D, D, "fp8", False, "cuda")
    pkv.pkv_scales_from_amax(src.k_pool.view(n_pages, H, P * D), False, dst.k_scale)
    pkv.pkv_scales_from_amax(src.v_pool.view(n_pages, H, P * D), False, dst.v_scale)
    sp = torch.randperm(n_pages, generator=g, device="cuda").to(torch.int32)
    dp = torch.randperm(n_pages, generator=g, device="cuda").to(torch.int32)
    tags = torch.randint(0, 2**31 - 1, (n_pages,), generator=g, device="cuda", dtype=torch.int32)
    for _ in range(3):
        pkv.pkv_requantize_pages(src, dst, sp, dp, tags)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(steps, 10)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        pkv.pkv_requantize_pages(src, dst, sp, dp, tags)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    moved = n_pages * H * P * D * 2 * 3
    return {"pages": n_pages, "ms": round(ms, 5), "bytes": moved,
            "gbs": round(moved / ms / 1e6, 2), "hbm_frac": round(moved / ms / 1e6 / HBM_PEAK_GBS, 4),
            "kernel": "requant_kernel (bf16 pages -> e4m3, tags)"}


def time_drafts(run, T: int, steps: int, warmup: int, read, dec_ms: float, flush):
    """pkv_decode_attn_drafts + pkv_combine over the Runner's resident cache:
    each request verifies its last T tokens together (query j sees the
    context up to L - T + j). The kernel reads the same cache bytes as a
    one-token decode; flops grow with T (QK^T and PV for T x Hq rows).
    Flushed like the step: the kernel's events after each flush."""
    import torch

    pkv, w, s = run.pkv, run.w, run.step
    g = torch.Generator(device="cuda").manual_seed(2029)
    q = torch.randn((w.batch, T, w.num_q_heads, w.head_dim_k), generator=g, device="cuda")
    q = q.to(torch.bfloat16)
    L = s.max_seq_len
    # the drafts kernel takes up to 128 pages per unit
    split = min(s.split_tokens, 128 * w.page_size)
    n_split = -(-L // split)
    o_part = torch.empty((w.batch, T * w.num_q_heads, n_split, w.head_dim_v),
                         dtype=torch.float32, device="cuda")
    lse_part = torch.empty((w.batch, T * w.num_q_heads, n_split), dtype=torch.float32,
                           device="cuda")
    out = torch.empty((w.batch, T * w.num_q_heads, w.head_dim_v), dtype=torch.bfloat16,
                      device="cuda")
    lse = torch.empty((w.batch, T * w.num_q_heads), dtype=torch.float32, device="cuda")
    abort = s.abort if s.verify else None

    def one(ev=None):
        if ev is not None:
            ev[0].record()
        pkv.pkv_decode_attn_drafts(run.cache, q, run.bt, run.lens, L, abort, w.sm_scale, split,
                                   o_part, lse_part)
        if ev is not None:
            ev[1].record()
        pkv.pkv_combine(o_part, lse_part, run.lens, split, L, abort, out, lse)

    for _ in range(warmup):
        flush()
        one()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        flush()
        one(e)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    nbytes = kv_bytes(w, 1, read)
    tokens = int(w.seq_lens[read].sum()) if read is not None else w.total_tokens
    flop = 2 * T * w.num_q_heads * (w.head_dim_k + w.head_dim_v) * tokens
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"q_len": T, "split_tokens": split, "decode_ms": round(ms, 5),
            "wall_ms_per_flushed_step": round((t1 - t0) * 1e3 / steps, 5),
            "kv_gbs": round(gbs, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
            "vs_q_len_single_token_decodes": round(T * dec_ms / ms, 3),
            "kernel": "decode_drafts_kernel (e4m3, MFMA 32x32x16 bf16/f16)"}


def time_int4(steps: int, warmup: int, layers: int = 16, n: int = 8192, k: int = 8192):
    """pkv_int4_linear over a stack of `layers` distinct n x k INT4 layers
    (codes + group scales: layers * (n*k/2 + n*k/64) bytes, above the MALL),
    one launch per layer, at batch 1 .. 64; beside it the same shapes as
    bf16 weights through torch's library GEMM. Each step is a captured HIP
    graph, replayed."""
    import torch

    import decode_attention_fp8_amd as pkv
    import workloads as W
    rows = []
    lays = [W.Int4Layer(f"int4_stack_{i}", 2000 + i, n, k, 64) for i in range(layers)]
    codes = [l.codes("cuda") for l in lays]
    scales = [l.scales("cuda") for l in lays]
    g = torch.Generator(device="cuda").manual_seed(2031)
    wbf = [torch.randn((n, k), generator=g, device="cuda").to(torch.bfloat16) for _ in range(layers)]
    w_bytes = layers * (n * k // 2 + (k // 128) * n * 2)
    for B in (1, 8, 16, 32, 64):
        x = lays[0].x("cuda")[:B].contiguous()
        y = torch.empty((B, n), dtype=torch.bfloat16, device="cuda")
        ws = pkv.int4_workspace(B, n, k, "cuda")

        def step_int4():
            for i in range(layers):
                pkv.pkv_int4_linear(x, codes[i], scales[i], y, ws)

        def step_bf16():
            for i in range(layers):
                torch.matmul(x, wbf[i].t(), out=y)

        res = {"batch": B}
        for name, fn in (("int4", step_int4), ("bf16", step_bf16)):
            # the step (one launch per layer) captured once and replayed, so
            # host launch costs do not enter the layer time
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(warmup):
                    fn()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn()
            for _ in range(warmup):
                graph.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / (steps * layers)
            del graph
            res[name] = {"ms_per_layer": round(ms, 5)}
        nb = w_bytes / layers + B * k * 2 + B * n * 2
        gbs = nb / (res["int4"]["ms_per_layer"] * 1e-3) / 1e9
        res["int4"].update({"gbs": round(gbs, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
        res["int4_speedup_over_bf16"] = round(res["bf16"]["ms_per_layer"] / res["int4"]["ms_per_layer"], 3)
        rows.append(res)
    del codes, scales, wbf
    torch.cuda.empty_cache()
    return {"layer": f"{n}x{k} INT4 (group 128, bf16 scales), {layers} distinct layers per step",
            "bytes_per_layer": w_bytes // layers,
            "kernel": "int4_lds_kernel (batch <= 8), int4_split_kernel + int4_sum_kernel (above)",
            "rows": rows}


def _oracle_unit(task):
    """One (request, kv head) unit of the oracle in a worker process: the
    unit's bf16 inputs are drawn first (not timed), then quantise K and V
    under the head's scales and run float64 attention for the head's query
    heads (timed). Returns (tokens, seconds)."""
    name, b, h, ks, vs, aborted = task
    from oracle import attention, quant, step
    if name not in _BUILT:
        _register_workloads()
        _BUILT[name] = _WORKLOADS[name]()
    w = _BUILT[name]
    x = step.bf16_bits_to_f64(w.k_bits(b, heads=[h]))[:, 0, :]
    y = step.bf16_bits_to_f64(w.v_bits(b, heads=[h]))[:, 0, :]
    q = step.bf16_bits_to_f64(w.q_bits()[b, h * w.group:(h + 1) * w.group])
    t = time.perf_counter()
    kk = quant.dequantize(quant.quantize(x, ks), ks)[:, None, :]
    vv = quant.dequantize(quant.quantize(y, vs), vs)[:, None, :]
    if not aborted:
        attention.attend(q, kk, vv, w.sm_scale)
    return int(w.seq_lens[b]), time.perf_counter() - t


def _worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    try:
        import torch
        torch.set_num_threads(1)
    except ImportError:
        pass


_WORKLOADS = {}  # name -> constructor of the workloads the baseline can sample
_BUILT = {}      # name -> workload, per process


def _register_workloads():
    import workloads as W
    _WORKLOADS.update({f"sweep_b{B}": (lambda B=B: W.sweep(B)) for B in W.SWEEP_BATCHES})
    _WORKLOADS.update({"gqa_b8": W.gqa, "long_b4": W.long_context})


def cpu_cores() -> int:
    """Host cores to use: this process's CPU affinity, at most 16 (a GPU machine's
    share for one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float = 6.0):
    """The oracle (tag check, quantise, float64 attention) on the host's
    cores, one process per core over (request, kv head) units, BLAS at one
    thread. Runs before the GPU is touched. A bounded sample: whole requests
    in order, as many as the first round of units (one per process, timed
    under full load) says fit in about budget_s of wall time; throughput =
    sample bytes / (summed unit time / processes). A unit's inputs are drawn
    before its clock starts."""
    import multiprocessing as mp

    import oracle
    from oracle import step
    _register_workloads()
    if w.name not in _WORKLOADS:
        return None
    n = cpu_cores()
    ks, vs = step.scales(w, "fp8")
    t = time.perf_counter()
    flags = oracle.verify.verify(w.page_tags, w.block_table, w.expected_tags, w.seq_lens,
                                 w.page_size)
    t_verify = time.perf_counter() - t
    H = w.num_kv_heads
    units = lambda reqs: [(w.name, b, h, ks[h], vs[h], bool(flags[b])) for b in reqs
                          for h in range(H)]
    ctx = mp.get_context("spawn")
    with ctx.Pool(n, initializer=_worker_init) as pool:
        # first, enough whole requests to give every process a unit; their
        # time under full load sets how many more requests fit the budget
        reqs = list(range(min(w.batch, -(-n // H))))
        res = pool.map(_oracle_unit, units(reqs), chunksize=1)
        per = sum(r[1] for r in res) / max(1, sum(r[0] for r in res))  # s per token and head
        est = sum(r[1] for r in res) / n
        more = []
        for b in range(len(reqs), w.batch):
            if est >= budget_s:
                break
            more.append(b)
            est += per * int(w.seq_lens[b]) * H / n
        if more:
            res += pool.map(_oracle_unit, units(more), chunksize=1)
        reqs += more
    tasks = units(reqs)
    busy = sum(r[1] for r in res) + t_verify
    tokens = sum(int(w.seq_lens[b]) for b in reqs)
    sample_bytes = tokens * w.num_kv_heads * (w.head_dim_k + w.head_dim_v)
    wall = busy / n
    return {"value": round(sample_bytes / wall / 1e9, 6), "unit": "GB/s", "cores": n,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {len(reqs)} of {w.batch} requests ({tokens} context tokens, all "
                      f"{w.num_kv_heads} kv heads, {len(tasks)} units on {n} processes): "
                      f"tag check of the batch, quantise K/V, float64 attention; "
                      f"{busy:.1f} s of unit time",
            "seq_steps_per_s": round(len(reqs) / wall, 4)}


def step_record(t: dict, nbytes: int, batch: int) -> dict:
    """Per-step figures from Runner.time: flushed median (headline) with its
    95% CI, warm median, decode kernel mean."""
    sm = summary(t)
    med = sm["flushed"]["median_ms"]
    return {"ms_per_step": med, "ci95_ms": sm["flushed"]["ci95_ms"],
            "kv_gbs": round(nbytes / (med * 1e-3) / 1e9, 2),
            "hbm_frac": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "seq_steps_per_s": round(batch / (med * 1e-3), 1),
            "graph_ms_per_step": sm["flushed_graph"]["median_ms"],
            "warm_ms_per_step": sm["warm"]["median_ms"],
            "warm_kv_gbs": round(nbytes / (sm["warm"]["median_ms"] * 1e-3) / 1e9, 2),
            "decode_ms": sm["decode"]["mean_ms"]}


DTYPE = ("e4m3 KV cache; QK^T bf16 x bf16 and P.V f16 x f16 on MFMA (codes convert exactly, "
         "numerators rounded to f16), f32 accumulation and softmax")
LATENT_DTYPE = ("e4m3 latent cache; QK^T bf16 x bf16 on MFMA (codes convert exactly in "
                "registers), P.V on scaled fp8 MFMA with V's codes as read and the numerators "
                "split into two e4m3 parts (eight significant bits), f32 accumulation and softmax")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "pkv measures one GPU; --gpus must be 1 (sharding is described, not run)"}))
        sys.exit(2)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch

    import workloads as W

    w = {"sweep": lambda: W.sweep(args.batch), "gqa": W.gqa, "long": W.long_context,
         "mla": W.mla}[args.workload]()
    # the oracle on the host's cores first, while no process has touched the GPU
    cpu = None
    if not args.no_cpu_baseline and not w.latent and not args.copy_calibration:
        cpu = cpu_baseline(w)

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return

    flush = Flusher()
    run = Runner(w, "fp8", args.split or None)
    t = run.time(args.steps, args.warmup, flush)
    sm = summary(t)
    ms = sm["flushed"]["median_ms"]
    dec_ms = sm["decode"]["mean_ms"]
    split = run.step.split_tokens
    # requests the step actually reads: those the tag check did not abort
    read = (run.step.abort.cpu().numpy() == 0) if run.step.verify else None
    n_aborted = 0 if read is None else int((~read).sum())
    tokens_read = int(w.seq_lens[read].sum()) if read is not None else w.total_tokens
    fp8_bytes = kv_bytes(w, 1, read)
    gbs = fp8_bytes / (ms * 1e-3) / 1e9
    dec_gbs = fp8_bytes / (dec_ms * 1e-3) / 1e9
    rec = {
        "metric": "FP8 paged decode-attn KV GB/s (% HBM peak) and seq-steps/s at B=1..64",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": LATENT_DTYPE if w.latent else DTYPE,
        "data": "synthetic (seeded counter-based bf16 N(0,1); lengths U[2048,32768])",
        "config": {"workload": f"{w.name}: {w.description}", "batch": w.batch,
                   "total_context_tokens": w.total_tokens, "split_tokens": split,
                   "aborted_requests": n_aborted, "context_tokens_read": tokens_read,
                   "kv_dtype": "e4m3", "kv_bytes": fp8_bytes},
        "flushed": True,
        "timing": {"method": f"median of {args.steps} steps, each after a {FLUSH_BYTES >> 20} MiB "
                             "write and read-back that evict the last-level cache; HIP events on its stream "
                             "around the step's launches (flushed_graph: around one replay of the "
                             "captured step; warm: replays back to back, no flush)",
                   **sm},
        "ci95_ms": sm["flushed"]["ci95_ms"],
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "seq_steps_per_s": round(w.batch / (ms * 1e-3), 1),
        "graph": {"ms_per_step": sm["flushed_graph"]["median_ms"],
                  "kv_gbs": round(fp8_bytes / (sm["flushed_graph"]["median_ms"] * 1e-3) / 1e9, 2)},
        "warm": {"ms_per_step": sm["warm"]["median_ms"],
                 "kv_gbs": round(fp8_bytes / (sm["warm"]["median_ms"] * 1e-3) / 1e9, 2)},
    }
    if w.latent:
        # the dense contraction bounds this kernel: QK^T over 576 dims and PV
        # over 512 for every (token, query head)
        flop = 2 * w.num_q_heads * (w.head_dim_k + w.head_dim_v) * tokens_read
        tflops = flop / (dec_ms * 1e-3) / 1e12
        rec["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK,
                           "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK, 4),
                           "traffic": measured_traffic(w, split),
                           "kernel": "pkv_decode_attn (latent e4m3: QK^T on bf16 MFMA, P.V on "
                                     "fp8 MFMA with two e4m3 products per multiply-add at the 5.0 "
                                     "PFLOP/s fp8 rate, so 2.5 PFLOP/s bounds both)",
                           "avg_ms": round(dec_ms, 5), "hbm_gbs": round(dec_gbs, 2),
                           "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4)}
    else:
        rec["roofline"] = {"bound": "hbm", "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic(w, split), "kernel": "pkv_decode_attn (e4m3)",
                           "avg_ms": round(dec_ms, 5)}
    if args.drafts:
        if w.latent or w.head_dim_k != 128 or w.head_dim_v != 128:
            rec["drafts"] = {"error": "the drafts path takes head dim 128 without a latent cache"}
        else:
            rec["drafts"] = time_drafts(run, args.drafts, args.steps, args.warmup, read, dec_ms,
                                        flush)
    del run
    torch.cuda.empty_cache()
    if not args.no_bf16:
        rb = Runner(w, "bf16", args.split or None)  # its own suggested split
        tb = rb.time(args.steps, args.warmup, flush)
        split_b = rb.step.split_tokens
        del rb
        torch.cuda.empty_cache()
        rec["bf16"] = {**step_record(tb, kv_bytes(w, 2, read), w.batch), "split_tokens": split_b}
        rec["fp8_speedup_over_bf16"] = round(rec["bf16"]["ms_per_step"] / ms, 4)
    if args.sweep:
        rows = []
        for B in W.SWEEP_BATCHES:
            ws = W.sweep(B)
            row = {"batch": B}
            for kv, e in (("fp8", 1), ("bf16", 2)):
                r = Runner(ws, kv, None)
                tr = r.time(max(20, args.steps), args.warmup, flush)
                nb = kv_bytes(ws, e, r.step.abort.cpu().numpy() == 0)
                row[kv] = {**step_record(tr, nb, B), "split_tokens": r.step.split_tokens}
                del r
                torch.cuda.empty_cache()
            row["fp8_speedup_over_bf16"] = round(row["bf16"]["ms_per_step"] / row["fp8"]["ms_per_step"], 4)
            rows.append(row)
        rec["sweep"] = rows
    if args.integrity:
        rows = []
        for B in (1, 2, 4, 8):
            wi = W.integrity_cost(B)
            on = Runner(wi, "fp8", None, verify=True)
            t_on = summary(on.time(max(50, args.steps), args.warmup, flush))
            del on
            off = Runner(wi, "fp8", None, verify=False)
            t_off = summary(off.time(max(50, args.steps), args.warmup, flush))
            del off
            torch.cuda.empty_cache()
            m_on, m_off = t_on["flushed"]["median_ms"], t_off["flushed"]["median_ms"]
            w_on, w_off = t_on["warm"]["median_ms"], t_off["warm"]["median_ms"]
            rows.append({"batch": B, "ms_verify_on": m_on, "ci95_on": t_on["flushed"]["ci95_ms"],
                         "ms_noop": m_off, "ci95_noop": t_off["flushed"]["ci95_ms"],
                         "overhead": round((m_on - m_off) / m_off, 4),
                         "warm_overhead": round((w_on - w_off) / w_off, 4)})
        rec["integrity_cost"] = rows
    if args.handoff:
        rec["handoff"] = time_handoff(args.steps)
    if args.row_scales and not w.latent:
        rr = Runner(w, "fp8", args.split or None, row_scales=True)
        tr = summary(rr.time(args.steps, args.warmup, flush))
        del rr
        torch.cuda.empty_cache()
        ms_r, dec_r = tr["flushed"]["median_ms"], tr["decode"]["mean_ms"]
        scale_bytes = int(w.seq_lens[read].sum() if read is not None else w.total_tokens) * \
            w.num_kv_heads * 2 * 4
        rec["row_scales"] = {
            "ms_per_step": round(ms_r, 5), "ci95_ms": tr["flushed"]["ci95_ms"],
            "decode_ms": round(dec_r, 5),
            "kv_gbs": round(fp8_bytes / (ms_r * 1e-3) / 1e9, 2),
            "decode_gbs_codes_and_scales": round((fp8_bytes + scale_bytes) / (dec_r * 1e-3) / 1e9, 2),
            "step_vs_static_scales": round(ms_r / ms, 4),
            "kernel": "decode_gqa_mfma_kernel<2, true>"}
    if args.int4:
        rec["int4_linear"] = time_int4(max(10, args.steps // 2), 3)
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
