"""Benchmark of the block-scaled int8 projection on one MI355X.

One step is one pass of the per-call prefill path over one batch of the large
prefill workload (M=8192, N=28672, K=8192, the largest single-GPU workload):
the BF16 -> int8 activation requant and the block-scaled int8 GEMM, the two
launches of the page's int8 prefill, through the C ABI.  `value` is 2*M*N*K /
step time (TOPS).  The NVFP4 -> int8 weight requant is a one-time cost (the page
runs it on a weight's first int8 prefill and keeps the result): it runs before
the timed steps and is reported on its own.  The dense-FFN prefill (gate+up
N=28672 K=4096 and down N=4096 K=14336 at M=4096) and the attention projection
(2048 x 4096 x 4096) are timed the same way and reported beside it; the decode
GEMV (M in {1,2,4,8}) is reported under "decode" in GB/s of algorithmic HBM
traffic.

Inputs are resident in HBM before timing.  Every timed iteration uses a
different set of buffers (rotating through enough sets that each set has left
the 256 MB Infinity Cache before it is used again).  Before the warm-up steps
the step runs untimed for ~100 ms (and every burst below for ~50 ms), so the
GPU's clocks have reached their steady state.  The step time is the wall
clock of the timed steps between two device synchronizations; inside the
timed region the two launches are bracketed by HIP events (timing-only
events without the system-scope fence, on the stream the launches use), which
gives the roofline's kernel duration.  Each kernel is also timed alone, back
to back over rotating buffers with one event pair around the whole burst
("us_burst"), which leaves out the per-launch event overhead that in-step
brackets carry.  The CPU oracle is timed beside it on a bounded sample (rank
0, one GPU only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "int8 block-scaled GEMM TOPS (prefill) + GEMV HBM GB/s, % of MI355X peak"
PEAK_INT8_TOPS = 5000.0        # MI355X dense int8 MFMA
PEAK_VALU_TOPS = 157.3 / 2                     # FP32 vector peak 157.3 TFLOP/s as FMA lane operations (T/s)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic.json")
GEMM_SOURCES = ["gemm.hip", "bsr_internal.h", "bsr_geometry.h"]
RQ_SOURCES = ["requant.hip", "bsr_internal.h", "bsr_geometry.h"]


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--decode-iters", type=int, default=100)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-oracle sample time")
    p.add_argument("--only", choices=["all", "prefill", "large", "split", "decode", "silu", "layouts", "copy"],
                   default="all",
                   help="large: the headline workload alone; prefill: it and the other prefill workloads; "
                        "copy: a plain 256 MiB device copy, the known-size reference for HBM byte counters")
    return p.parse_args()


def _source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "block_scaled_precision_requant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _traffic(kernel, source_files):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the summary is missing or the kernel source changed since it was taken."""
    try:
        with open(PROFILE_COUNTERS) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != _source_digest(source_files):
        return None
    return rec.get("bytes_per_launch")


class HipEvent:
    """A HIP event for timing only, recorded on a given stream: created with
    hipEventDisableSystemFence, so recording it skips the system-scope cache
    writeback and invalidation that a default event (torch's) performs, which
    would otherwise stall the stream between the kernels it brackets."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            # the HIP runtime torch loaded (the one that owns its streams)
            with open("/proc/self/maps") as f:
                paths = [ln.split()[-1] for ln in f if "libamdhip64.so" in ln]
            cls._hip = ctypes.CDLL(paths[0] if paths else "libamdhip64.so")
        return cls._hip

    def __init__(self):
        self.h = ctypes.c_void_p()
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(self.h), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags: {rc}")

    def record(self, stream):
        rc = self._runtime().hipEventRecord(self.h, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord: {rc}")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both complete: synchronize first)."""
        ms = ctypes.c_float()
        rc = self._runtime().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime: {rc}")
        return ms.value

    def __del__(self):
        try:
            if self._hip is not None and self.h:
                self._hip.hipEventDestroy(self.h)
        except Exception:  # interpreter shutdown: the runtime may already be gone
            pass


def settle(fn, seconds):
    """Run fn(0), fn(1), ... untimed for about `seconds` of wall time.  Under a
    sustained load the GPU's clocks take ~35 ms to reach their steady state
    (the prefill step falls from ~137 to ~112 us over that time), so every
    timed region is preceded by this."""
    import torch
    t0, i = time.perf_counter(), 0
    while True:
        for _ in range(16):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def main():
    args = _args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              f"the multi-GPU sharding is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import oracle
    from block_scaled_precision_requant_amd import bsr, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    rec = {}

    if args.only == "copy":
        # known-size reference for rocprofv3 FETCH_SIZE / WRITE_SIZE: each copy
        # reads and writes exactly 256 MiB
        src = torch.ones(256 * 2 ** 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "copies": 5}), flush=True)
        return

    def dev_t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    def burst(fn, reps):
        """Average duration of `reps` back-to-back launches fn(i) (one event pair),
        after ~50 ms of the same launches untimed."""
        settle(fn, 0.05)
        e0, e1 = HipEvent(), HipEvent()
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    # ------------------------------------------------------------ prefill
    # Each prefill workload: its buffers in `nsets` full copies (NVFP4 weight,
    # int8 weight, activations, activation scratch, output), so back-to-back
    # launches never find their operands in the Infinity Cache; the weight
    # requant runs on every set first (the one-time step), then the bursts.
    def prefill_sets(proj):
        M, N, K = proj.m, proj.n, proj.k
        packed, e4m3 = proj.weight()
        a_bits = proj.activations()
        set_bytes = (N * K // 2 + N * K // 16 + N * K + N * K // 8 + 2 * M * K + M * K + M * K // 8 + 2 * M * N)
        nsets = max(2, int(np.ceil(1.0 * 2 ** 30 / set_bytes)))
        wp, we, a = dev_t(packed), dev_t(e4m3), dev_t(a_bits.view(np.int16))
        sets = []
        for i in range(nsets):
            sets.append(dict(
                wp=wp if i == 0 else wp.clone(), we=we if i == 0 else we.clone(),
                a=a if i == 0 else a.clone(),
                w_i8=torch.empty((N, K), dtype=torch.int8, device=dev),
                w_s=torch.empty((N, K // 32), dtype=torch.float32, device=dev),
                a_i8=torch.empty((M, K), dtype=torch.int8, device=dev),
                a_s=torch.empty((M, K // 32), dtype=torch.float32, device=dev),
                out=torch.empty((M, N), dtype=torch.int16, device=dev)))
        return sets, packed, e4m3, a_bits

    def requant_w(st, scale2):
        bsr.requant_w_nvfp4_int8(st["wp"], st["we"], scale2, st["w_i8"], st["w_s"], stream=stream)

    def requant_a(st):
        bsr.requant_a_int8(st["a"], st["a_i8"], st["a_s"], stream=stream)

    def gemm(st):
        bsr.int8_gemm_blockscaled(st["a_i8"], st["w_i8"], st["a_s"], st["w_s"], st["out"], stream=stream)

    def prefill_bursts(proj, sets, reps):
        """Per-launch times of the weight requant (one-time), the activation
        requant, the GEMM and the two-launch prefill, each a burst over the sets."""
        M, N, K = proj.m, proj.n, proj.k
        ns = len(sets)
        scale2 = float(proj.scale2)
        ops = 2.0 * M * N * K
        bytes_w = N * K * (0.5 + 1 / 16 + 1 + 1 / 8)
        bytes_a = M * K * (2 + 1 + 1 / 8)
        b_w = burst(lambda i: requant_w(sets[i % ns], scale2), reps)
        b_a = burst(lambda i: requant_a(sets[i % ns]), reps)
        b_g = burst(lambda i: gemm(sets[i % ns]), reps)

        def pair(i):  # the two-launch prefill: activation requant, then the GEMM
            requant_a(sets[i % ns])
            gemm(sets[i % ns])
        b_ag = burst(pair, reps)
        return {
            "requant_w_nvfp4_int8": dict(one_time=True, us_burst=b_w * 1e6, mb=bytes_w / 1e6,
                                         hbm_bytes_counters=_traffic(f"requant_w_kernel|{proj.name}", RQ_SOURCES),
                                         gbs=bytes_w / b_w / 1e9, frac_hbm=bytes_w / b_w / 1e9 / PEAK_HBM_GBS),
            "requant_a_int8": dict(us_burst=b_a * 1e6, mb=bytes_a / 1e6, gbs=bytes_a / b_a / 1e9,
                                   hbm_bytes_counters=_traffic(f"requant_a_kernel|{proj.name}", RQ_SOURCES),
                                   frac_hbm=bytes_a / b_a / 1e9 / PEAK_HBM_GBS),
            "int8_gemm_blockscaled": dict(us_burst=b_g * 1e6, tops=ops / b_g / 1e12,
                                          hbm_bytes_counters=_traffic(f"gemm_kernel|{proj.name}", GEMM_SOURCES),
                                          frac_int8=ops / b_g / 1e12 / PEAK_INT8_TOPS),
            "requant_a_plus_gemm": dict(us_burst=b_ag * 1e6, tops=ops / b_ag / 1e12,
                                        frac_int8=ops / b_ag / 1e12 / PEAK_INT8_TOPS),
        }

    def check_rows(proj, st, a_bits, rows, ow, osw):
        """The GPU output rows of set `st` against the oracle (same seeded inputs)."""
        from oracle.compare import check_bf16
        oa, osa = oracle.requant_a(a_bits[rows])
        y, t = oracle.gemm_ref(oa, ow, osa, osw)
        got = st["out"][torch.as_tensor(rows, device=dev)].cpu().numpy().view(np.uint16)
        res = check_bf16(got, y, t, proj.k)
        return dict(rows=int(len(rows)), ok=res.ok, failures=res.failures, needed_fp32_sum_bound=res.needed_ii,
                    max_rel_err=res.max_rel_err)

    def band_rows(m, per_band, seed):
        """`per_band` seeded rows in every 128-row tile band of the output."""
        rng = np.random.default_rng(seed)
        rows = []
        for t0 in range(0, m, 128):
            h = min(128, m - t0)
            rows += [t0 + int(o) for o in rng.choice(h, size=min(per_band, h), replace=False)]
        return np.array(sorted(rows), dtype=np.int64)

    head = None
    if args.only in ("all", "prefill", "large"):
        # ---- the headline: the large prefill, one step = requant_a + GEMM
        proj = inputs.workload("large").projections[0]
        M, N, K = proj.m, proj.n, proj.k
        sets, packed, e4m3, a_bits = prefill_sets(proj)
        nsets = len(sets)
        scale2 = float(proj.scale2)
        ops = 2.0 * M * N * K
        # the one-time weight requant: once per set, the first launch timed on its own
        e0, e1 = HipEvent(), HipEvent()
        e0.record(stream)
        requant_w(sets[0], scale2)
        e1.record(stream)
        for st in sets[1:]:
            requant_w(st, scale2)
        torch.cuda.synchronize()
        t_w_first = e0.elapsed_time(e1) * 1e-3

        def step(st, ev=None):
            if ev is not None:
                ev[0].record(stream)
            requant_a(st)
            if ev is not None:
                ev[1].record(stream)
            gemm(st)
            if ev is not None:
                ev[2].record(stream)

        settle(lambda i: step(sets[i % nsets]), 0.1)
        for i in range(args.warmup):
            step(sets[i % nsets])
        evs = [[HipEvent(), HipEvent(), HipEvent()] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(sets[i % nsets], evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        t_a = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
        t_g = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
        ms_per_step = wall / args.steps * 1e3
        kern = prefill_bursts(proj, sets, max(6, 2 * nsets))
        kern["requant_w_nvfp4_int8"]["us_first_launch"] = t_w_first * 1e6
        kern["int8_gemm_blockscaled"].update(us_in_step_mean=t_g.mean() * 1e6,
                                             us_in_step_median=float(np.median(t_g)) * 1e6,
                                             us_in_step_min=t_g.min() * 1e6,
                                             tops_in_step=ops / t_g.mean() / 1e12)
        kern["requant_a_int8"].update(us_in_step_mean=t_a.mean() * 1e6)
        # parity of the timed outputs: one step on set 0, then one seeded row in
        # every 128-row tile band (64 rows) against the oracle
        step(sets[0])
        torch.cuda.synchronize()
        ow, osw = oracle.requant_w(packed, e4m3, proj.scale2)
        parity = check_rows(proj, sets[0], a_bits, band_rows(M, 1, 1004), ow, osw)
        head = dict(proj=proj, ms_per_step=ms_per_step, value_tops=ops / (ms_per_step * 1e-3) / 1e12,
                    kernels=kern, parity=parity, buffer_sets=nsets, packed=packed, e4m3=e4m3, a_bits=a_bits,
                    ow=ow, osw=osw)
        del sets
        torch.cuda.empty_cache()

    if args.only in ("all", "prefill"):
        # ---- the dense FFN's two projections and the attention projection, timed the same way
        others = {}
        for proj in inputs.workload("dense_ffn").projections + inputs.workload("attn_proj").projections:
            sets, packed_o, e4m3_o, a_o = prefill_sets(proj)
            for st in sets:
                requant_w(st, float(proj.scale2))
            torch.cuda.synchronize()
            kern_o = prefill_bursts(proj, sets, max(20, 2 * len(sets)))
            gemm(sets[0])
            torch.cuda.synchronize()
            ow_o, osw_o = oracle.requant_w(packed_o, e4m3_o, proj.scale2)
            par_o = check_rows(proj, sets[0], a_o, band_rows(proj.m, 1, 1000 + proj.seed), ow_o, osw_o)
            others[proj.name] = dict(m=proj.m, n=proj.n, k=proj.k, buffer_sets=len(sets), kernels=kern_o,
                                     parity=par_o)
            del sets, ow_o, osw_o
            torch.cuda.empty_cache()
        rec["other_prefill"] = others

    # ------------------------------------------------------------ K split across workgroups
    # The rows between decode and prefill at the down projection's width (n = 4096,
    # k = 14336): the default path (no workspace) against the K split into a caller
    # workspace and through the allocation-free entry point's static scratch.
    if args.only in ("all", "split"):
        sp = {}
        dproj = [q for q in inputs.workload("decode").projections if q.name == "decode_m8_n4096_k14336"][0]
        wp, we = dproj.weight()
        n, k = dproj.n, dproj.k
        w_i8 = torch.empty((n, k), dtype=torch.int8, device=dev)
        w_s = torch.empty((n, k // 32), dtype=torch.float32, device=dev)
        bsr.requant_w_nvfp4_int8(dev_t(wp), dev_t(we), float(dproj.scale2), w_i8, w_s)
        ncopy = max(2, int(np.ceil(2 ** 30 / (n * k * 1.125))))
        copies = [(w_i8.clone(), w_s.clone()) for _ in range(ncopy)]
        rng_sp = np.random.default_rng(5)
        for m in (17, 32, 64, 128, 192):
            a_bits = inputs.bf16_normal(rng_sp, m, k)
            a_i8 = torch.empty((m, k), dtype=torch.int8, device=dev)
            a_s = torch.empty((m, k // 32), dtype=torch.float32, device=dev)
            bsr.requant_a_int8(dev_t(a_bits.view(np.int16)), a_i8, a_s)
            out = torch.empty((m, n), dtype=torch.int16, device=dev)
            need = bsr.int8_gemm_blockscaled_ws_bytes(m, n, k)
            ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device=dev) if need else None
            t_def = burst(lambda i: bsr.int8_gemm_blockscaled(a_i8, copies[i % ncopy][0], a_s, copies[i % ncopy][1],
                                                              out, stream=stream), args.decode_iters)
            t_ws = burst(lambda i: bsr.int8_gemm_blockscaled_ws(a_i8, copies[i % ncopy][0], a_s, copies[i % ncopy][1],
                                                                out, ws, stream=stream), args.decode_iters)
            t_na = burst(lambda i: bsr.int8_gemm_blockscaled_noalloc(a_i8, copies[i % ncopy][0], a_s,
                                                                     copies[i % ncopy][1], out, stream=stream),
                         args.decode_iters)
            alg = n * k * 1.125 + m * k * 1.125 + 2 * m * n
            sp[f"m{m}_n{n}_k{k}"] = dict(workspace_bytes=need, default_us_burst=t_def * 1e6,
                                         ws_us_burst=t_ws * 1e6, noalloc_us_burst=t_na * 1e6,
                                         tops_best=2.0 * m * n * k / min(t_def, t_ws) / 1e12,
                                         gbs_best=alg / min(t_def, t_ws) / 1e9)
        del copies
        torch.cuda.empty_cache()
        rec["split"] = sp

    # ------------------------------------------------------------ decode
    if args.only in ("all", "decode"):
        dec = {}
        for p in inputs.workload("decode").projections:
            wp, we = p.weight()
            a = p.activations()
            w_i8 = torch.empty((p.n, p.k), dtype=torch.int8, device=dev)
            w_s = torch.empty((p.n, p.k // 32), dtype=torch.float32, device=dev)
            bsr.requant_w_nvfp4_int8(dev_t(wp), dev_t(we), float(p.scale2), w_i8, w_s)
            wbytes = p.n * p.k * 1.125
            ncopy = max(2, int(np.ceil(2 ** 30 / wbytes)))
            copies = [(w_i8.clone(), w_s.clone()) for _ in range(ncopy)]
            a_dev = dev_t(a.view(np.int16))
            a_i8 = torch.empty((p.m, p.k), dtype=torch.int8, device=dev)
            a_s = torch.empty((p.m, p.k // 32), dtype=torch.float32, device=dev)
            out = torch.empty((p.m, p.n), dtype=torch.int16, device=dev)
            bsr.requant_a_int8(a_dev, a_i8, a_s)
            it = args.decode_iters
            t_v = burst(lambda i: bsr.int8_gemm_blockscaled(a_i8, copies[i % ncopy][0], a_s, copies[i % ncopy][1],
                                                            out, stream=stream), it)

            def requant_and_gemv(i):
                bsr.requant_a_int8(a_dev, a_i8, a_s, stream=stream)
                bsr.int8_gemm_blockscaled(a_i8, copies[i % ncopy][0], a_s, copies[i % ncopy][1], out, stream=stream)
            t_qv = burst(requant_and_gemv, it)
            # the path-invariant GEMV (one FP32 chain per output, in the GEMM's order)
            t_inv = burst(lambda i: bsr.int8_gemm_blockscaled_ex(a_i8, copies[i % ncopy][0], a_s, copies[i % ncopy][1],
                                                                 out, path=bsr.PATH_INVARIANT, stream=stream), it)
            alg = p.n * p.k * 1.125 + p.m * p.k * 1.125 + 2 * p.m * p.n
            del copies
            # W4A16: the same product straight from the NVFP4 weight (0.5625 B per weight)
            w4bytes = p.n * p.k * (0.5 + 1 / 16)
            ncopy4 = max(2, int(np.ceil(2 ** 30 / w4bytes)))
            wp_d, we_d = dev_t(wp), dev_t(we)
            copies4 = [(wp_d.clone(), we_d.clone()) for _ in range(ncopy4)]
            out4 = torch.empty((p.m, p.n), dtype=torch.int16, device=dev)
            t_4 = burst(lambda i: bsr.w4a16_gemv(a_dev, copies4[i % ncopy4][0], copies4[i % ncopy4][1],
                                                 float(p.scale2), out4, stream=stream), it)
            alg4 = w4bytes + p.m * p.k * 2 + 2 * p.m * p.n
            cpu_dec = {}
            if not args.no_cpu_baseline:
                # the oracle beside it (host threads): activation requant + GEMV reference on
                # the weight requantized once beforehand, and the W4A16 reference
                ow, osw = oracle.requant_w(wp, we, p.scale2)
                t0 = time.perf_counter()
                oa, osa = oracle.requant_a(a)
                oracle.gemm_ref(oa, ow, osa, osw)
                t_o = time.perf_counter() - t0
                t0 = time.perf_counter()
                oracle.w4a16_ref(a, wp, we, p.scale2)
                t_o4 = time.perf_counter() - t0
                cpu_dec = dict(cpu_oracle_requant_a_plus_gemv_us=t_o * 1e6, cpu_oracle_w4a16_us=t_o4 * 1e6,
                               cpu_cores=oracle.max_threads())
            dec[p.name] = dict(m=p.m, n=p.n, k=p.k, gemv_us_burst=t_v * 1e6, **cpu_dec,
                               gemv_gbs=alg / t_v / 1e9, gemv_frac_hbm=alg / t_v / 1e9 / PEAK_HBM_GBS,
                               requant_a_plus_gemv_us_burst=t_qv * 1e6,
                               invariant_gemv_us_burst=t_inv * 1e6,
                               invariant_gemv_frac_hbm=alg / t_inv / 1e9 / PEAK_HBM_GBS,
                               w4a16_us_burst=t_4 * 1e6, w4a16_gbs=alg4 / t_4 / 1e9,
                               w4a16_frac_hbm=alg4 / t_4 / 1e9 / PEAK_HBM_GBS)
            del copies4
            torch.cuda.empty_cache()
        gbs = [d["gemv_gbs"] for d in dec.values()]
        rec["decode"] = dict(cases=dec, gemv_gbs_mean=float(np.mean(gbs)),
                             gemv_frac_hbm_mean=float(np.mean(gbs)) / PEAK_HBM_GBS)

    # ------------------------------------------------------------ fused SiLU requant
    if args.only in ("all", "silu"):
        src = inputs.silu_mul_input()
        g_bits, u_bits = src.gate(), src.up()
        sbytes = src.m * src.k * (2 + 2 + 1 + 1 / 8)
        nset = max(2, int(np.ceil(2 ** 30 / sbytes)))
        ssets = [dict(g=dev_t(g_bits.view(np.int16)), u=dev_t(u_bits.view(np.int16)),
                      q=torch.empty((src.m, src.k), dtype=torch.int8, device=dev),
                      s=torch.empty((src.m, src.k // 32), dtype=torch.float32, device=dev))
                 for _ in range(nset)]
        t_s = burst(lambda i: bsr.silu_mul_requant_int8(ssets[i % nset]["g"], ssets[i % nset]["u"],
                                                        ssets[i % nset]["q"], ssets[i % nset]["s"],
                                                        stream=stream), max(10, 2 * nset))
        rec["silu"] = dict(workload=f"SiLU(gate) * up -> int8 per 32, M={src.m} I={src.k}",
                           us_burst=t_s * 1e6, gbs=sbytes / t_s / 1e9,
                           frac_hbm=sbytes / t_s / 1e9 / PEAK_HBM_GBS)
        if not args.no_cpu_baseline:
            t0 = time.perf_counter()
            oracle.silu_mul_requant(g_bits, u_bits)
            rec["silu"]["cpu_oracle_us"] = (time.perf_counter() - t0) * 1e6
            rec["silu"]["cpu_cores"] = oracle.max_threads()
        del ssets
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ other activation layouts
    if args.only in ("all", "layouts"):
        lay = {}
        # on the attention projection's activation (2048 x 4096) and weight (4096 x 4096)
        lp = inputs.workload("attn_proj").projections[0]
        M, N, K = lp.m, lp.n, lp.k
        packed, e4m3 = lp.weight()
        a_bits = lp.activations()
        scale2 = float(lp.scale2)
        qbytes = {32: M * K * (2 + 1 + 4 / 32), 128: M * K * (2 + 1 + 4 / 128), 0: M * K * 3 + 4 * M}
        nq = max(2, int(np.ceil(2 ** 30 / (M * K * 3))))
        a_copies = [dev_t(a_bits.view(np.int16)) for _ in range(nq)]
        q_buf = torch.empty((M, K), dtype=torch.uint8, device=dev)
        for fmt, fname in ((bsr.FMT_INT8, "int8"), (bsr.FMT_E4M3, "e4m3")):
            for g in (32, 128, 0):
                s_buf = torch.empty((M, 1 if g == 0 else K // g), dtype=torch.float32, device=dev)
                t_q = burst(lambda i: bsr.quantize_act(a_copies[i % nq], q_buf, s_buf, group=g, fmt=fmt,
                                                       stream=stream), max(20, 2 * nq))
                gname = "row" if g == 0 else str(g)
                lay[f"quantize_act_{fname}_g{gname}"] = dict(us_burst=t_q * 1e6, gbs=qbytes[g] / t_q / 1e9,
                                                              frac_hbm=qbytes[g] / t_q / 1e9 / PEAK_HBM_GBS)
        del a_copies
        w_i8 = torch.empty((N, K), dtype=torch.int8, device=dev)
        w_s = torch.empty((N, K // 32), dtype=torch.float32, device=dev)
        bsr.requant_w_nvfp4_int8(dev_t(packed), dev_t(e4m3), scale2, w_i8, w_s)
        a_dev = dev_t(a_bits.view(np.int16))
        out = torch.empty((M, N), dtype=torch.int16, device=dev)
        for g in (32, 128, 0):
            s_buf = torch.empty((M, 1 if g == 0 else K // g), dtype=torch.float32, device=dev)
            bsr.quantize_act(a_dev, q_buf, s_buf, group=g, stream=stream)
            t_g = burst(lambda i: bsr.int8_gemm_blockscaled_agroup(q_buf.view(torch.int8), w_i8, s_buf, g, w_s, out,
                                                                   stream=stream), 20)
            gname = "row" if g == 0 else str(g)
            lay[f"gemm_agroup_g{gname}"] = dict(us_burst=t_g * 1e6, tops=2.0 * M * N * K / t_g / 1e12)
        del w_i8, w_s
        # decode GEMV with grouped activation scales (M=8, N=4096, K=14336)
        p = [q for q in inputs.workload("decode").projections if q.name == "decode_m8_n4096_k14336"][0]
        wp, we = p.weight()
        w_i8 = torch.empty((p.n, p.k), dtype=torch.int8, device=dev)
        w_s = torch.empty((p.n, p.k // 32), dtype=torch.float32, device=dev)
        bsr.requant_w_nvfp4_int8(dev_t(wp), dev_t(we), float(p.scale2), w_i8, w_s)
        ncopy = max(2, int(np.ceil(2 ** 30 / (p.n * p.k * 1.125))))
        copies = [(w_i8.clone(), w_s.clone()) for _ in range(ncopy)]
        xa = dev_t(p.activations().view(np.int16))
        xq = torch.empty((p.m, p.k), dtype=torch.uint8, device=dev)
        xo = torch.empty((p.m, p.n), dtype=torch.int16, device=dev)
        for g in (32, 128, 0):
            xs = torch.empty((p.m, 1 if g == 0 else p.k // g), dtype=torch.float32, device=dev)
            bsr.quantize_act(xa, xq, xs, group=g, stream=stream)
            t_v = burst(lambda i: bsr.int8_gemm_blockscaled_agroup(xq.view(torch.int8), copies[i % ncopy][0], xs, g,
                                                                   copies[i % ncopy][1], xo, stream=stream),
                        args.decode_iters)
            alg = p.n * p.k * 1.125 + p.m * p.k + xs.numel() * 4 + 2 * p.m * p.n
            gname = "row" if g == 0 else str(g)
            lay[f"gemv_agroup_g{gname}_{p.name}"] = dict(us_burst=t_v * 1e6, gbs=alg / t_v / 1e9,
                                                        frac_hbm=alg / t_v / 1e9 / PEAK_HBM_GBS)
        del copies
        torch.cuda.empty_cache()
        rec["layouts"] = lay

    # ------------------------------------------------------------ context
    # achievable streaming bandwidth: a plain device copy (torch's), read + write
    # counted, 512 MiB each way, ten copies between one event pair
    if args.only in ("all", "prefill"):
        src = torch.ones(512 * 2 ** 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        settle(lambda i: dst.copy_(src), 0.05)
        e0, e1 = HipEvent(), HipEvent()
        e0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        t_c = e0.elapsed_time(e1) * 1e-3 / 10
        rec["copy_context"] = dict(bytes_per_copy=2 * src.numel(), us=t_c * 1e6,
                                   gbs=2 * src.numel() / t_c / 1e9,
                                   frac_hbm=2 * src.numel() / t_c / 1e9 / PEAK_HBM_GBS)
        del src, dst
        torch.cuda.empty_cache()
        # a plain streaming read (read_probe.hip: 16-byte loads in a grid-stride
        # loop, libbsr_read.so), per launch, at the decode weights' sizes and at
        # 1 GiB, buffers rotated over >= 1 GiB: what one launch of that many bytes
        # costs here, launch and ramp included (best of three grid sizes)
        rlib = ctypes.CDLL(os.path.join(os.path.dirname(bsr.LIB_PATH), "libbsr_read.so"))
        rlib.read_probe.restype = ctypes.c_int
        rlib.read_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32,
                                    ctypes.c_void_p]
        sink = torch.empty(4096, dtype=torch.int32, device=dev)
        reads = {}
        for label, nbytes in (("33MB", 33_554_432), ("66MB", 67_108_864), ("1GiB", 2 ** 30)):
            nbuf = max(2, -(-2 ** 30 // nbytes))
            bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
            best = None
            for grid in (1024, 2048, 4096):
                def read(i, grid=grid):
                    rc = rlib.read_probe(ctypes.c_void_p(bufs[i % nbuf].data_ptr()), nbytes,
                                         ctypes.c_void_p(sink.data_ptr()), grid, ctypes.c_void_p(stream.cuda_stream))
                    assert rc == 0
                t_r = burst(read, 50 if nbytes < 2 ** 30 else 10)
                if best is None or t_r < best[0]:
                    best = (t_r, grid)
            reads[label] = dict(bytes=nbytes, us=best[0] * 1e6, gbs=nbytes / best[0] / 1e9,
                                frac_hbm=nbytes / best[0] / 1e9 / PEAK_HBM_GBS, grid=best[1])
            del bufs
            torch.cuda.empty_cache()
        rec["read_context"] = reads

    # ------------------------------------------------------------ CPU oracle
    # The oracle (as is, OpenMP over rows) on the host threads, on the headline
    # workload: the one-time weight requant in full (timed on its own), and the
    # step -- the activation requant in full plus the GEMM reference on seeded rows
    # (two in every 128-row tile band, 128 rows) extrapolated linearly to all M rows.
    cpu = None
    if not args.no_cpu_baseline and head is not None:
        proj = head["proj"]
        M, N, K = proj.m, proj.n, proj.k
        packed, e4m3, a_bits = head["packed"], head["e4m3"], head["a_bits"]
        cores = oracle.max_threads()
        t0 = time.perf_counter()
        ow, osw = oracle.requant_w(packed, e4m3, proj.scale2)
        t_rw = time.perf_counter() - t0
        t0 = time.perf_counter()
        oa, osa = oracle.requant_a(a_bits)
        t_ra = time.perf_counter() - t0
        rows = band_rows(M, 2, 2004)
        t0 = time.perf_counter()
        oracle.gemm_ref(oa, ow, osa, osw, rows=rows)
        t_rows = time.perf_counter() - t0
        t_step = t_ra + t_rows * M / len(rows)
        cpu = dict(value=2.0 * M * N * K / t_step / 1e12, unit="TOPS", cores=cores, kind="oracle",
                   sample=(f"large prefill {M}x{N}x{K}: activation requant of all {M} rows ({t_ra:.2f} s) + "
                           f"GEMM reference on {len(rows)} of {M} rows, two seeded rows in every 128-row band "
                           f"({t_rows:.2f} s), extrapolated linearly to all rows; the one-time weight requant "
                           f"({t_rw:.2f} s, all {N} rows) is reported apart"),
                   seconds_per_step_extrapolated=t_step, weight_requant_seconds=t_rw,
                   cpu_model=_cpu_model())
        # the same oracle on one thread: 64 activation rows and 4 GEMM rows,
        # extrapolated linearly to the whole step
        oracle.set_threads(1)
        try:
            t0 = time.perf_counter()
            oracle.requant_a(a_bits[:64])
            t1_a = (time.perf_counter() - t0) * M / 64
            t0 = time.perf_counter()
            oracle.gemm_ref(oa, ow, osa, osw, rows=rows[:4])
            t1_g = (time.perf_counter() - t0) * M / 4
        finally:
            oracle.set_threads(cores)
        t1 = t1_a + t1_g
        cpu["single_thread"] = dict(value=2.0 * M * N * K / t1 / 1e12, unit="TOPS", cores=1,
                                    sample="activation requant on 64 of M rows, GEMM reference on 4 of M rows, "
                                           "each extrapolated linearly",
                                    seconds_per_step_extrapolated=t1)

    line = {
        "metric": METRIC,
        "value": head["value_tops"] if head else None,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"] if head else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "large prefill M=8192 N=28672 K=8192 (A ~ N(0,1) BF16 with 8 fixed columns x100, "
                               "NVFP4 W scales 2^U{-6..4}, scale2 = fl32(1/448))",
                   "m": 8192, "n": 28672, "k": 8192,
                   "step": "requant_a_int8 + int8_gemm_blockscaled (the weight requantized once, before the "
                           "timed steps, and timed apart)"},
    }
    if head:
        proj = head["proj"]
        M, N, K = proj.m, proj.n, proj.k
        g = head["kernels"]["int8_gemm_blockscaled"]
        line["roofline"] = {"bound": "mfma", "achieved": g["tops_in_step"], "peak": PEAK_INT8_TOPS,
                            "unit": "TOPS", "frac": g["tops_in_step"] / PEAK_INT8_TOPS,
                            "traffic": _traffic("gemm_kernel|large", GEMM_SOURCES),
                            "kernel": "gemm_kernel (int8_gemm_blockscaled, m > 16), large prefill"}
        # The same kernel against the vector ALU, which bounds it: the exact
        # per-block FP32 rescale is one int32 -> FP32 conversion and one FMA per
        # output and 32-wide K block; peak = the FP32 vector peak, 157.3 TFLOP/s,
        # counted as FMA lane operations (78.6 T/s).  The SQ counters of this
        # kernel show wave64 VALU instructions issuing faster than 16 lanes per
        # cycle, so 16 lanes x 4 SIMDs x 256 CUs x 2.4 GHz is no ceiling.
        alu_ops = 2.0 * M * N * (K // 32)
        alu = alu_ops / (g["us_in_step_mean"] * 1e-6) / 1e12
        line["roofline_alu"] = {"bound": "alu", "achieved": alu, "peak": PEAK_VALU_TOPS,
                                "unit": "T lane-ops/s", "frac": alu / PEAK_VALU_TOPS,
                                "work": "int32->FP32 conversion + FMA per output and K block"}
        line["kernels"] = head["kernels"]
        line["parity"] = head["parity"]
        line["buffer_sets"] = head["buffer_sets"]
    if "other_prefill" in rec:
        line["other_prefill"] = rec["other_prefill"]
    if cpu:
        line["cpu_baseline"] = cpu
    if "split" in rec:
        line["split_k"] = rec["split"]
    if "decode" in rec:
        line["decode"] = rec["decode"]
    if "silu" in rec:
        line["silu_mul_requant"] = rec["silu"]
    if "layouts" in rec:
        line["activation_layouts"] = rec["layouts"]
    if "copy_context" in rec:
        line["copy_context"] = rec["copy_context"]
    if "read_context" in rec:
        line["read_context"] = rec["read_context"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
