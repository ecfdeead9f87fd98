"""Benchmark: MLA decode over a paged latent KV cache on one MI355X.

One step = one pass of the whole decode path over one batch: the split-KV plan
(mla_get_metadata), the attention kernel (mla_decode_attn) and the LSE
combine (mla_decode_combine).  Inputs are resident in HBM before timing.

The headline line is measured on the memory-bound workload (batch 128 x 4096
tokens, h_q = 16); the same JSON line carries the other workloads
(compute-bound h_q = 128, FP8 cache, long context) under "workloads", each
with TFLOP/s, GB/s and roofline fractions, plus the oracle timed on the host
cores as a CPU baseline.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
# MI355X dense bf16 MFMA: 256 CUs x 4096 FLOP per clock x 2.4 GHz
PEAK_BF16_TFLOPS = 2517.0
FLUSH_BYTES = 1 << 30        # written, then another buffer of this size read, before each
                             # flushed iteration (> the 256 MB MALL and the 8 x 4 MB L2s)
METRIC = "MLA decode TFLOPS + HBM GB/s (fraction of MI355X peak), h_q=16 and h_q=128"


class CacheEvict:
    """Leaves the caches holding none of the workload's lines and no dirty
    lines: FLUSH_BYTES written to one scratch buffer, then FLUSH_BYTES of
    another read.  The read evicts the written lines, so their write-back
    happens here and not inside the timed call that follows (a write alone
    leaves up to the MALL's size of dirty lines, whose write-back made the
    memory-bound step about 50% slower)."""

    def __init__(self, torch, device):
        self.torch = torch
        self.w = torch.empty((FLUSH_BYTES,), dtype=torch.uint8, device=device)
        self.r = torch.ones((FLUSH_BYTES // 8,), dtype=torch.int64, device=device)

    def __call__(self, k):
        self.w.fill_(k & 0xFF)
        self.r.sum()

    def free(self):
        del self.w, self.r


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="membound")
    p.add_argument("--extra",
                   default="computebound,fp8,longctx,tiny,kvwrite,sparse,sparse16,fp8_accuracy,ceilings",
                   help="comma list of further workloads to measure ('' for none)")
    p.add_argument("--flush", action="store_true",
                   help="every workload also reports steps timed one by one after a cache "
                        "eviction (1 GiB written, another 1 GiB read; membound, tiny and "
                        "sparse always do)")
    p.add_argument("--flush-iters", type=int, default=30)
    p.add_argument("--cpu-baseline", type=int, default=1)
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--sweep", action="store_true",
                   help="only run the shape sweep (one JSON line per shape)")
    p.add_argument("--sweep-fp8", action="store_true",
                   help="only run the shape sweep over FP8 caches")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run plain 1 GiB device copies (to scale HBM counters)")
    return p.parse_args()


class Runner:
    """Device inputs, a preallocated plan / workspace / outputs, and a step."""

    def __init__(self, name, inputs=None):
        """`name`: a workload of workloads.CONFIGS, or a label when `inputs`
        gives (q, kcache, block_table, seqlens, s_q, h_q, causal, scale, fp8)."""
        import torch
        import mla_paged_kv_fwd_amd as mla
        import workloads as W

        self.torch, self.mla, self.name = torch, mla, name
        (self.q, self.kc, self.bt, self.sl, self.s_q, self.h_q, self.causal, self.scale,
         self.fp8) = inputs if inputs is not None else W.make_config_device(name)
        seqlens = self.sl.cpu().numpy()
        self.batch = seqlens.shape[0]
        self.bytes = W.algorithmic_bytes(seqlens, self.s_q, self.h_q, self.fp8)
        self.flops = W.algorithmic_flops(seqlens, self.s_q, self.h_q, self.causal)
        self.num_parts = mla.default_num_parts(self.s_q, self.h_q, fp8=self.fp8, batch=self.batch,
                                               max_seqlen=int(seqlens.max()))
        dev = self.q.device
        self.meta = torch.empty((self.num_parts, mla.META_INTS), dtype=torch.int32, device=dev)
        self.split_base = torch.empty((self.batch + 1,), dtype=torch.int32, device=dev)
        ws = mla.workspace_bytes(self.batch, self.s_q, self.h_q, self.num_parts)
        self.ws = torch.empty((ws,), dtype=torch.uint8, device=dev)
        self.out = torch.empty((self.batch, self.s_q, self.h_q, mla.D_V), dtype=torch.bfloat16,
                               device=dev)
        self.lse = torch.empty((self.batch, self.s_q, self.h_q), dtype=torch.float32, device=dev)
        lib = mla.lib()
        self._plan_args = (self.sl.data_ptr(), self.batch, self.s_q, self.h_q, self.num_parts,
                           self.meta.data_ptr(), self.split_base.data_ptr())
        self._attn_args = (self.q.data_ptr(), self.kc.data_ptr(), 1 if self.fp8 else 0,
                           self.kc.shape[0], self.bt.data_ptr(), self.bt.shape[1],
                           self.sl.data_ptr(), self.batch, self.s_q, self.h_q, float(self.scale),
                           int(self.causal), self.meta.data_ptr(), self.split_base.data_ptr(),
                           self.num_parts, self.ws.data_ptr(), self.ws.numel(),
                           self.out.data_ptr(), self.lse.data_ptr())
        self._comb_args = (self.split_base.data_ptr(), self.batch, self.s_q, self.h_q,
                           self.num_parts, self.ws.data_ptr(), self.ws.numel(),
                           self.out.data_ptr(), self.lse.data_ptr())
        self.lib = lib

    def step(self, events=None):
        stream = self.torch.cuda.current_stream()
        s = stream.cuda_stream
        if events is not None:
            events[0].record(stream)
        st = self.lib.mla_get_metadata(*self._plan_args, s)
        if events is not None:
            events[1].record(stream)
        st |= self.lib.mla_decode_attn(*self._attn_args, s)
        if events is not None:
            events[2].record(stream)
        st |= self.lib.mla_decode_combine(*self._comb_args, s)
        if events is not None:
            events[3].record(stream)
        if st != 0:
            raise RuntimeError(f"libmla call failed in {self.name}")

    def measure(self, steps, warmup, graph=True):
        """Times `steps` whole steps between two events (nothing else inside
        the timed region); then, in a second pass of `steps` steps, the plan,
        attention and combine calls separately with events on the same
        stream; then `steps` attention launches back to back between two
        events (the kernel's average launch duration, the roofline's time)."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            self.step()
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_step = e0.elapsed_time(e1) / steps
        wall_ms_step = (t1 - t0) * 1e3 / steps
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for k in range(steps):
            self.step(evs[k])
        torch.cuda.synchronize()
        plan = np.mean([e[0].elapsed_time(e[1]) for e in evs])
        attn = np.mean([e[1].elapsed_time(e[2]) for e in evs])
        comb = np.mean([e[2].elapsed_time(e[3]) for e in evs])
        pct_step = percentiles([e[0].elapsed_time(e[3]) * 1e3 for e in evs])
        pct_attn = percentiles([e[1].elapsed_time(e[2]) * 1e3 for e in evs])
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(steps):
            if self.lib.mla_decode_attn(*self._attn_args, stream.cuda_stream) != 0:
                raise RuntimeError(f"libmla call failed in {self.name}")
        a1.record(stream)
        torch.cuda.synchronize()
        kernel = a0.elapsed_time(a1) / steps
        n_split = int(self.split_base[-1].item())
        graph_ms = None
        if graph:
            try:  # a reported extra: the timed step above does not depend on it
                graph_ms = self.measure_graph(steps)
            except Exception as exc:  # noqa: BLE001
                print(f"[bench] {self.name}: graph replay not measured ({exc})", file=sys.stderr)
        return dict(ms_per_step=ms_step, wall_ms_per_step=wall_ms_step, plan_us=plan * 1e3,
                    attn_us=attn * 1e3, combine_us=comb * 1e3, attn_kernel_us=kernel * 1e3,
                    split_slots=n_split, graph_ms_per_step=graph_ms,
                    step_us_pct=pct_step, attn_us_pct=pct_attn)

    def measure_flushed(self, iters):
        """`iters` steps timed one by one, each after a CacheEvict (the 256 MB
        MALL and the L2s hold none of the workload and nothing dirty), with
        events around the whole step and around the attention call: p10 /
        median / p90 in microseconds."""
        torch = self.torch
        flush = CacheEvict(torch, self.q.device)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(iters)]
        for k in range(iters):
            flush(k)
            self.step(evs[k])
        torch.cuda.synchronize()
        res = dict(iters=iters, flush_bytes=FLUSH_BYTES,
                   step_us=percentiles([e[0].elapsed_time(e[3]) * 1e3 for e in evs]),
                   attn_us=percentiles([e[1].elapsed_time(e[2]) * 1e3 for e in evs]))
        res["gbs_median"] = round(self.bytes / res["step_us"]["p50"] / 1e3, 1)
        res["tflops_median"] = round(self.flops / res["step_us"]["p50"] / 1e6, 1)
        flush.free()
        return res

    def measure_graph(self, steps):
        """The same step (plan, attention, combine) captured once in a HIP
        graph and replayed `steps` times between two events.  The first
        replay's output must equal the eager step's bit for bit."""
        torch = self.torch
        self.step()
        torch.cuda.synchronize()
        ref_out, ref_lse = self.out.clone(), self.lse.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        self.out.zero_()
        self.lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not (torch.equal(self.out.view(torch.int16), ref_out.view(torch.int16))
                and torch.equal(self.lse, ref_lse)):
            raise RuntimeError(f"graph replay differs from the eager step in {self.name}")
        for _ in range(10):
            g.replay()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def report(self, m):
        s = m["ms_per_step"] * 1e-3
        a = m["attn_kernel_us"] * 1e-6
        gbs, tfl = self.bytes / s / 1e9, self.flops / s / 1e12
        gbs_k, tfl_k = self.bytes / a / 1e9, self.flops / a / 1e12
        bound = "hbm" if self.bytes / (PEAK_HBM_GBS * 1e9) >= self.flops / (PEAK_BF16_TFLOPS * 1e12) else "mfma"
        return dict(
            us_per_step=round(m["ms_per_step"] * 1e3, 2),
            us_per_step_graph=(None if m["graph_ms_per_step"] is None
                               else round(m["graph_ms_per_step"] * 1e3, 2)),
            wall_us_per_step=round(m["wall_ms_per_step"] * 1e3, 2), plan_us=round(m["plan_us"], 2),
            attn_us=round(m["attn_us"], 2), combine_us=round(m["combine_us"], 2),
            attn_kernel_us=round(m["attn_kernel_us"], 2),
            step_us_pct=m["step_us_pct"], attn_us_pct=m["attn_us_pct"],
            split_slots=m["split_slots"], num_parts=self.num_parts,
            alg_bytes=self.bytes, alg_flops=self.flops,
            gbs=round(gbs, 1), tflops=round(tfl, 1),
            attn_gbs=round(gbs_k, 1), attn_tflops=round(tfl_k, 1),
            hbm_frac=round(gbs / PEAK_HBM_GBS, 4), mfma_frac=round(tfl / PEAK_BF16_TFLOPS, 4),
            bound=bound,
            roofline_frac=round(max(gbs / PEAK_HBM_GBS, tfl / PEAK_BF16_TFLOPS), 4))


def percentiles(xs):
    """p10, median and p90 of a list of times (microseconds)."""
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 2), "p50": round(float(np.median(a)), 2),
            "p90": round(float(np.percentile(a, 90)), 2)}


def ceilings(steps):
    """Measured ceilings of the part, in the same run as the decode legs: a
    plain streaming read of 2 GiB (16-byte loads, several grid sizes, the
    best kept) and back-to-back bf16 MFMA loops (16x16x32 and 32x32x16, one
    or two waves per SIMD, the best kept).  Launches timed back to back
    between two events, after three untimed ones."""
    import ctypes

    import torch
    import mla_paged_kv_fwd_amd as mla

    lib = ctypes.CDLL(mla.CEILING_LIB_PATH)
    lib.mla_ceiling_blocks.argtypes = [ctypes.c_int]
    lib.mla_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p]
    lib.mla_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p]
    lib.mla_ceiling_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.mla_ceiling_mfma_flops.restype = ctypes.c_double
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream

    def timed(launch, n):
        for _ in range(3):
            if launch() != 0:
                raise RuntimeError("ceiling launch failed")
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(n):
            launch()
        a1.record(stream)
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) / n * 1e-3  # seconds per launch

    nbytes = 2 << 30
    buf = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    read = {}
    for bpc in (2, 4, 8, 16):
        sink = torch.empty((lib.mla_ceiling_blocks(bpc) * 256,), dtype=torch.int32, device="cuda")
        t = timed(lambda: lib.mla_ceiling_stream_read(buf.data_ptr(), nbytes, bpc,
                                                      sink.data_ptr(), s), max(steps, 10))
        read[f"{bpc}_per_cu"] = round(nbytes / t / 1e9, 1)
    del buf
    mfma = {}
    for shape, name in ((0, "16x16x32"), (1, "32x32x16")):
        for bpc in (1, 2):
            iters = 20000
            sink = torch.empty((lib.mla_ceiling_blocks(bpc) * 256,), dtype=torch.float32,
                               device="cuda")
            t = timed(lambda: lib.mla_ceiling_mfma(shape, iters, bpc, sink.data_ptr(), s),
                      max(steps // 2, 5))
            mfma[f"{name}_{bpc}_wave_per_simd"] = round(
                lib.mla_ceiling_mfma_flops(shape, iters, bpc) / t / 1e12, 1)
    best_read = max(read.values())
    best_16 = max(v for k, v in mfma.items() if k.startswith("16x16x32"))
    best_32 = max(v for k, v in mfma.items() if k.startswith("32x32x16"))
    torch.cuda.empty_cache()
    return dict(hbm_read_gbs=best_read, hbm_read_frac=round(best_read / PEAK_HBM_GBS, 4),
                mfma_16x16x32_tflops=best_16, mfma_32x32x16_tflops=best_32,
                mfma_frac=round(max(best_16, best_32) / PEAK_BF16_TFLOPS, 4),
                read_by_grid=read, mfma_by_shape=mfma)


def kv_write_bench(steps, warmup):
    """The cache writer on the FP8 workload's cache written whole, as a prefill
    would: 64 requests x 16384 rows of 576 bf16 values quantised into 656-byte
    records (the kernel reads 1152 B and writes 656 B per row).  Also the
    decode append of the same batch (2 rows per request).  Launches timed back
    to back between two events on the launch stream."""
    import torch
    import mla_paged_kv_fwd_amd as mla
    import workloads as W

    batch, length = 64, 16384
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    pages = length // W.PAGE
    perm = torch.randperm(batch * pages, generator=g, device="cuda").to(torch.int32)
    bt = perm.reshape(batch, pages).contiguous()
    sl = torch.full((batch,), length, dtype=torch.int32, device="cuda")
    kc = torch.zeros((batch * pages, W.PAGE, W.FP8_RECORD), dtype=torch.uint8, device="cuda")
    k_new = torch.randn((batch, length, W.D_QK), generator=g, device="cuda").to(torch.bfloat16)
    stream = torch.cuda.current_stream()
    lib = mla.lib()

    def timed(rows):
        src = k_new if rows == length else k_new[:, length - rows:].contiguous()  # kept alive
        args = (src.data_ptr(), batch, rows, bt.data_ptr(), pages, sl.data_ptr(), kc.data_ptr(),
                kc.shape[0], stream.cuda_stream)
        for _ in range(warmup):
            lib.mla_kv_cache_write_fp8(*args)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(steps):
            if lib.mla_kv_cache_write_fp8(*args) != 0:
                raise RuntimeError("mla_kv_cache_write_fp8 failed")
        a1.record(stream)
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) / steps * 1e3

    us = timed(length)
    rows = batch * length
    alg = rows * (2 * W.D_QK + W.FP8_RECORD) + batch * pages * 4 + batch * 4
    us_append = timed(2)
    return dict(kernel="kv_write_kernel<true>", rows=rows, us=round(us, 2), alg_bytes=alg,
                gbs=round(alg / us / 1e3, 1), hbm_frac=round(alg / us / 1e3 / PEAK_HBM_GBS, 4),
                bound="hbm", append_rows=2 * batch, append_us=round(us_append, 2))


SWEEP_BATCH = (8, 32, 128)
SWEEP_LEN = (1024, 4096, 16384)
SWEEP_HQ = (16, 32, 64, 128)
SWEEP_SQ = (1, 2, 4)


def sweep(steps, warmup, fp8=False):
    """Shape sweep over batch x sequence length x h_q x s_q (causal when
    s_q > 1), bf16 or FP8 cache, every request at the same length.  One JSON line per
    shape: the whole step and the attention kernel back to back, with their
    throughput and the kernel's fraction of its roofline."""
    import math

    import torch
    import workloads as W

    for batch in SWEEP_BATCH:
        for length in SWEEP_LEN:
            for h_q in SWEEP_HQ:
                for s_q in SWEEP_SQ:
                    sl = np.full(batch, length, dtype=np.int32)
                    q, kc, bt, slt = W.make_device_inputs(sl, s_q, h_q, fp8, seed=batch + length + h_q)
                    r = Runner(f"sweep b{batch} L{length} h{h_q} s{s_q}",
                               (q, kc, bt, slt, s_q, h_q, s_q > 1, 1.0 / math.sqrt(W.D_QK), fp8))
                    rep = r.report(r.measure(steps, warmup, graph=False))
                    a = rep["attn_kernel_us"] * 1e-6
                    frac = max(rep["alg_bytes"] / a / (PEAK_HBM_GBS * 1e9),
                               rep["alg_flops"] / a / (PEAK_BF16_TFLOPS * 1e12))
                    print(json.dumps(dict(batch=batch, seqlen=length, h_q=h_q, s_q=s_q, fp8=fp8,
                                          step_us=rep["us_per_step"],
                                          attn_kernel_us=rep["attn_kernel_us"],
                                          attn_gbs=rep["attn_gbs"], attn_tflops=rep["attn_tflops"],
                                          bound=rep["bound"], attn_roofline_frac=round(frac, 4),
                                          split_slots=rep["split_slots"])), flush=True)
                    del r, q, kc, bt, slt
                    torch.cuda.empty_cache()


def sparse_bench(steps, warmup, h_q=128, flush_iters=30):
    """Sparse decode over the FP8 workload's cache (64 requests x 16384
    tokens, s_q 1; h_q 128, or the first h_q heads of its queries): each query
    token attends to 2048 distinct listed tokens.  The whole call (token ids, plan, decode, combine) between two
    events, launches back to back; FLOPs = 2 * h_q * (576 + 512) per listed
    token and row; bytes = the listed records read once, plus q, out, lse and
    the lists."""
    import math

    import torch
    import mla_paged_kv_fwd_amd as mla
    import workloads as W

    q, kc, bt, sl, s_q, h_all, _, scale, _ = W.make_config_device("fp8")
    q = q[:, :, :h_q].contiguous()
    batch, length, topk = q.shape[0], int(sl[0].item()), 2048
    g = torch.Generator(device="cuda")
    g.manual_seed(79)
    idx = torch.argsort(torch.rand((batch, s_q, length), generator=g, device="cuda"), dim=-1)[
        ..., :topk].to(torch.int32).contiguous()
    num_parts = mla.default_num_parts(1, h_q, fp8=True, sparse=True)
    ws = torch.empty((mla.sparse_workspace_bytes(batch, s_q, h_q, topk, num_parts, fp8=True),),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((batch, s_q, h_q, W.D_V), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device="cuda")
    lib = mla.lib()
    stream = torch.cuda.current_stream()
    args = (q.data_ptr(), kc.data_ptr(), 1, kc.shape[0], bt.data_ptr(), bt.shape[1], idx.data_ptr(),
            topk, batch, s_q, h_q, float(scale), num_parts, ws.data_ptr(), ws.numel(),
            out.data_ptr(), lse.data_ptr(), stream.cuda_stream)
    for _ in range(warmup):
        lib.mla_decode_sparse(*args)
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(steps):
        if lib.mla_decode_sparse(*args) != 0:
            raise RuntimeError("mla_decode_sparse failed")
    a1.record(stream)
    torch.cuda.synchronize()
    us = a0.elapsed_time(a1) / steps * 1e3
    # the same call timed one by one after a CacheEvict: the listed records
    # (86 MB) would otherwise stay in the 256 MB MALL between calls
    flush = CacheEvict(torch, "cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(flush_iters)]
    for k, (f0, f1) in enumerate(evs):
        flush(k)
        f0.record(stream)
        lib.mla_decode_sparse(*args)
        f1.record(stream)
    torch.cuda.synchronize()
    flushed = percentiles([f0.elapsed_time(f1) * 1e3 for f0, f1 in evs])
    flush.free()
    rows = batch * s_q
    flops = 2 * h_q * (W.D_QK + W.D_V) * topk * rows
    alg = rows * topk * (W.FP8_RECORD + 4) + rows * h_q * (2 * W.D_QK + 2 * W.D_V + 4)
    res = dict(shape=f"batch {batch} x {length}, s_q {s_q}, h_q {h_q}, fp8 cache, {topk} listed tokens",
               us=round(us, 2), us_flushed=flushed, alg_flops=flops, alg_bytes=alg,
               tflops=round(flops / us / 1e6, 1),
               tflops_flushed_median=round(flops / flushed["p50"] / 1e6, 1),
               mfma_frac=round(flops / us / 1e6 / PEAK_BF16_TFLOPS, 4),
               gbs=round(alg / us / 1e3, 1))
    del q, kc, bt, sl, idx, ws, out, lse
    torch.cuda.empty_cache()
    return res


def fp8_accuracy():
    """FP8 cache against bf16 cache on the same latent, across shapes: h_q in
    {16, 64, 128} x L in {4096, 16384, 65536}, s_q 1, 2^20 cached tokens per
    shape (batch = 2^20 / L; h_q 128 at L 16384 is the FP8 workload's shape).
    N(0,1) rows rounded to bf16 are written once as bf16 rows and once as FP8
    records by the cache writer and both are decoded with the same queries.
    Reports how far the FP8 result moves from the bf16 one: a property of the
    format and its quantiser, not a parity check (the GPU tests set this shift
    beside the oracle's own on sampled rows)."""
    import math

    import torch
    import mla_paged_kv_fwd_amd as mla
    import workloads as W

    res = []
    for h_q in (16, 64, 128):
        for length in (4096, 16384, 65536):
            batch = (1 << 20) // length
            g = torch.Generator(device="cuda")
            g.manual_seed(78 + h_q + length)
            pages = length // W.PAGE
            bt = torch.randperm(batch * pages, generator=g, device="cuda").to(torch.int32).reshape(
                batch, pages).contiguous()
            sl = torch.full((batch,), length, dtype=torch.int32, device="cuda")
            rows = torch.randn((batch, length, W.D_QK), generator=g, device="cuda").to(torch.bfloat16)
            q = torch.randn((batch, 1, h_q, W.D_QK), generator=g, device="cuda").to(torch.bfloat16)
            kc16 = torch.empty((batch * pages, W.PAGE, W.D_QK), dtype=torch.bfloat16, device="cuda")
            kc8 = torch.empty((batch * pages, W.PAGE, W.FP8_RECORD), dtype=torch.uint8, device="cuda")
            mla.kv_cache_write(rows, bt, sl, kc16)
            mla.kv_cache_write(rows, bt, sl, kc8, fp8=True)
            del rows
            scale = 1.0 / math.sqrt(W.D_QK)
            o16, l16 = mla.decode(q, kc16, bt, sl, scale, False)
            o8, l8 = mla.decode(q, kc8, bt, sl, scale, False, fp8=True)
            torch.cuda.synchronize()
            d = o8.float() - o16.float()
            res.append(dict(h_q=h_q, L=length, batch=batch,
                            out_max_abs=round(d.abs().max().item(), 6),
                            out_rel_l2=round((d.norm() / o16.float().norm()).item(), 6),
                            out_ref_max_abs=round(o16.float().abs().max().item(), 6),
                            lse_max_abs=round((l8 - l16).abs().max().item(), 6),
                            lse_mean_abs=round((l8 - l16).abs().mean().item(), 6)))
            del kc16, kc8, o16, o8, l16, l8, d
            torch.cuda.empty_cache()
    return res


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary under profiles/, if the kernel's source still
    hashes to what was profiled; otherwise None."""
    import glob
    import hashlib

    here = os.path.dirname(os.path.abspath(__file__))
    for path in sorted(glob.glob(os.path.join(here, "profiles", "*.md"))):
        fields = {}
        for ln in open(path):
            if ln.startswith("traffic_") and ":" in ln:
                k, v = ln.split(":", 1)
                fields[k.strip()] = v.strip()
        if fields.get("traffic_kernel") != kernel or fields.get("traffic_workload") != workload:
            continue
        # the profiled sources: one sha256 over their bytes in the listed order
        h = hashlib.sha256()
        for rel in fields.get("traffic_source", "").split():
            src = os.path.join(here, rel)
            if not os.path.isfile(src):
                return None
            h.update(open(src, "rb").read())
        if h.hexdigest() != fields.get("traffic_source_sha256"):
            return None
        return int(fields["traffic_bytes_per_launch"])
    return None


def cpu_baseline(name, seconds):
    """The oracle on a bounded sample of the workload: whole requests of the
    same shape, doubling the sample until about `seconds` of wall time."""
    import oracle
    import workloads as W

    cfg = W.CONFIGS[name]
    rng = np.random.Generator(np.random.PCG64(cfg["seed"]))
    all_sl = W.config_seqlens(name, rng)
    n = 1
    while True:
        sl = all_sl[:n]
        case = W.make_case(sl, cfg["s_q"], cfg["h_q"], seed=cfg["seed"] + 1000, causal=cfg["causal"],
                           fp8=cfg["fp8"])
        rows = oracle.all_rows(case.batch, case.s_q, case.h_q)
        t0 = time.perf_counter()
        _, _, threads = oracle.decode_rows(case.q, case.cache, case.kind, case.block_table,
                                           case.seqlens, case.scale, case.causal, rows)
        dt = time.perf_counter() - t0
        if dt >= seconds / 2 or n >= len(all_sl):
            break
        n = min(len(all_sl), n * 2)
    # the whole workload fits the budget: repeat it and take the mean time
    reps = 1
    total = dt
    while n >= len(all_sl) and total < seconds / 2:
        t0 = time.perf_counter()
        oracle.decode_rows(case.q, case.cache, case.kind, case.block_table, case.seqlens,
                           case.scale, case.causal, rows)
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    b = W.algorithmic_bytes(sl, cfg["s_q"], cfg["h_q"], cfg["fp8"])
    f = W.algorithmic_flops(sl, cfg["s_q"], cfg["h_q"], cfg["causal"])
    return dict(value=round(b / dt / 1e9, 4), unit="GB/s", cores=int(threads), kind="oracle",
                sample=f"{n} of {len(all_sl)} requests ({cfg['desc']}), all rows, "
                       f"{dt:.2f} s per pass, mean of {reps} pass(es)",
                tflops=round(f / dt / 1e12, 6), seconds=round(dt, 3))


def roofline(rep, workload, ceil=None):
    """Roofline object for the dominant kernel of the workload's step: the
    attention kernel, timed with events on the stream it runs on.  With the
    ceilings leg measured, also its fraction of the part's measured rate."""
    import workloads as W

    cfg = W.CONFIGS[workload]
    rows = cfg["s_q"] * cfg["h_q"]
    if rows < 32:
        kernel = "decode_rowgroup_kernel<%s, false>" % ("true" if cfg["fp8"] else "false")
    elif rows == 128 and not cfg["fp8"]:
        kernel = "decode_rows128_kernel"
    else:
        kernel = "decode_rows64_fp8_kernel<false>" if cfg["fp8"] else "decode_rows64_kernel<false>"
    traffic = measured_traffic(kernel, workload)
    if rep["bound"] == "hbm":
        achieved, peak, unit = rep["attn_gbs"], PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = rep["attn_tflops"], PEAK_BF16_TFLOPS, "TFLOP/s"
    res = {"bound": rep["bound"], "achieved": achieved, "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel}
    if ceil:
        measured = (ceil["hbm_read_gbs"] if rep["bound"] == "hbm" else
                    max(ceil["mfma_16x16x32_tflops"], ceil["mfma_32x32x16_tflops"]))
        res["peak_measured"] = measured
        res["frac_of_measured"] = round(achieved / measured, 4)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones((n,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 3}))
        return
    if args.sweep or args.sweep_fp8:
        sweep(args.steps, args.warmup, fp8=args.sweep_fp8)
        return
    always_flushed = ("membound", "tiny")
    main_r = Runner(args.workload)
    m = main_r.measure(args.steps, args.warmup)
    rep = main_r.report(m)
    if args.flush or args.workload in always_flushed:
        rep["flushed"] = main_r.measure_flushed(args.flush_iters)
    print(f"[bench] {args.workload}: {json.dumps(rep)}", file=sys.stderr, flush=True)
    workloads = {args.workload: rep}
    del main_r
    for name in [x for x in args.extra.split(",") if x]:
        if name in ("kvwrite", "fp8_accuracy", "sparse", "sparse16", "ceilings"):
            rep_x = (kv_write_bench(args.steps, args.warmup) if name == "kvwrite" else
                     sparse_bench(args.steps, args.warmup, flush_iters=args.flush_iters)
                     if name == "sparse" else
                     sparse_bench(args.steps, args.warmup, h_q=16, flush_iters=args.flush_iters)
                     if name == "sparse16" else
                     ceilings(args.steps) if name == "ceilings" else
                     fp8_accuracy())
            print(f"[bench] {name}: {json.dumps(rep_x)}", file=sys.stderr, flush=True)
            workloads[name] = rep_x
            torch.cuda.empty_cache()
            continue
        r = Runner(name)
        rep_x = r.report(r.measure(args.steps, args.warmup))
        if args.flush or name in always_flushed:
            rep_x["flushed"] = r.measure_flushed(args.flush_iters)
        if name == "tiny":  # a latency figure: the whole step and its calls, in microseconds
            rep_x = {k: rep_x[k] for k in ("us_per_step", "plan_us", "attn_us", "combine_us",
                                           "attn_kernel_us", "step_us_pct", "flushed",
                                           "alg_bytes", "alg_flops")}
            rep_x["bound"] = "latency"
        print(f"[bench] {name}: {json.dumps(rep_x)}", file=sys.stderr, flush=True)
        workloads[name] = rep_x
        del r
        torch.cuda.empty_cache()
    ceil = workloads.get("ceilings")
    if ceil:  # every throughput workload's kernel also against the measured ceilings
        for name, r in workloads.items():
            if isinstance(r, dict) and "attn_gbs" in r:
                r["attn_frac_of_measured"] = round(max(
                    r["attn_gbs"] / ceil["hbm_read_gbs"],
                    r["attn_tflops"] / max(ceil["mfma_16x16x32_tflops"],
                                           ceil["mfma_32x32x16_tflops"])), 4)
    head = workloads[args.workload]
    attn_gbs = head["attn_gbs"]
    line = {
        "metric": METRIC,
        "value": head["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {W.CONFIGS[args.workload]['desc']}, page 64",
                   "batch": int(len(W.CONFIGS[args.workload]['seqlens'])) if not isinstance(
                       W.CONFIGS[args.workload]['seqlens'], tuple) else 64,
                   "parallelism": "single GPU"},
        "roofline": roofline(head, args.workload, ceil),
        "workloads": workloads,
    }
    if args.cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
