"""Benchmark of the block-scaled int8 projection on one MI355X.

One step is one pass of the whole prefill path over one batch of the prefill
attention-projection workload (M=2048, N=4096, K=4096): the NVFP4 -> int8
weight requant, the BF16 -> int8 activation requant and the block-scaled int8
GEMM, all through the C ABI.  `value` is 2*M*N*K / step time (TOPS).  The
decode GEMV (M in {1,2,4,8}) is timed in the same run on its own workload and
reported under "decode" in GB/s of algorithmic HBM traffic.

Inputs are resident in HBM before timing.  Every timed iteration uses a
different set of buffers (rotating through enough sets that each set has left
the 256 MB Infinity Cache before it is used again).  Before the warm-up steps
the step runs untimed for ~100 ms (and every burst below for ~50 ms), so the
GPU's clocks have reached their steady state.  The step time is the wall
clock of the timed steps between two device synchronizations; inside the
timed region only the GEMM launches are bracketed by HIP events (timing-only
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
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12   # non-packed FP32 VALU lane operations per second (T)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--decode-iters", type=int, default=100)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-oracle sample time")
    p.add_argument("--only", choices=["all", "prefill", "decode", "silu", "layouts", "copy"], default="all",
                   help="copy: a plain 256 MiB device copy, the known-size reference for HBM byte counters")
    return p.parse_args()


def _source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "block_scaled_precision_requant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(kernel, source_files, launches_bytes_alg):
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

    # ------------------------------------------------------------ prefill
    proj = inputs.workload("attn_proj").projections[0]
    M, N, K = proj.m, proj.n, proj.k
    packed, e4m3 = proj.weight()
    a_bits = proj.activations()
    set_bytes = (N * K // 2 + N * K // 16 + N * K + N * K // 8 + 2 * M * K + M * K + M * K // 8 + 2 * M * N)
    nsets = max(2, int(np.ceil(1.0 * 2 ** 30 / set_bytes)))
    sets = []
    for _ in range(nsets):
        sets.append(dict(
            wp=dev_t(packed), we=dev_t(e4m3), a=dev_t(a_bits.view(np.int16)),
            w_i8=torch.empty((N, K), dtype=torch.int8, device=dev),
            w_s=torch.empty((N, K // 32), dtype=torch.float32, device=dev),
            a_i8=torch.empty((M, K), dtype=torch.int8, device=dev),
            a_s=torch.empty((M, K // 32), dtype=torch.float32, device=dev),
            out=torch.empty((M, N), dtype=torch.int16, device=dev)))
    scale2 = float(proj.scale2)

    def step(s, ev=None):
        bsr.requant_w_nvfp4_int8(s["wp"], s["we"], scale2, s["w_i8"], s["w_s"], stream=stream)
        bsr.requant_a_int8(s["a"], s["a_i8"], s["a_s"], stream=stream)
        if ev is not None:
            ev[0].record(stream)
        bsr.int8_gemm_blockscaled(s["a_i8"], s["w_i8"], s["a_s"], s["w_s"], s["out"], stream=stream)
        if ev is not None:
            ev[1].record(stream)

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

    if args.only in ("all", "prefill"):
        settle(lambda i: step(sets[i % nsets]), 0.1)
        for i in range(args.warmup):
            step(sets[i % nsets])
        evs = [[HipEvent(), HipEvent()] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(sets[i % nsets], evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        t_g = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
        ms_per_step = wall / args.steps * 1e3
        ops = 2.0 * M * N * K
        gemm_tops = ops / t_g.mean() / 1e12
        bytes_w = N * K * (0.5 + 1 / 16 + 1 + 1 / 8)
        bytes_a = M * K * (2 + 1 + 1 / 8)
        reps = max(20, nsets)
        b_w = burst(lambda i: bsr.requant_w_nvfp4_int8(sets[i % nsets]["wp"], sets[i % nsets]["we"], scale2,
                                                       sets[i % nsets]["w_i8"], sets[i % nsets]["w_s"],
                                                       stream=stream), reps)
        b_a = burst(lambda i: bsr.requant_a_int8(sets[i % nsets]["a"], sets[i % nsets]["a_i8"],
                                                 sets[i % nsets]["a_s"], stream=stream), reps)
        b_g = burst(lambda i: bsr.int8_gemm_blockscaled(sets[i % nsets]["a_i8"], sets[i % nsets]["w_i8"],
                                                        sets[i % nsets]["a_s"], sets[i % nsets]["w_s"],
                                                        sets[i % nsets]["out"], stream=stream), reps)

        def prefill_pair(i):  # the two-launch prefill: activation requant, then the GEMM
            st = sets[i % nsets]
            bsr.requant_a_int8(st["a"], st["a_i8"], st["a_s"], stream=stream)
            bsr.int8_gemm_blockscaled(st["a_i8"], st["w_i8"], st["a_s"], st["w_s"], st["out"], stream=stream)
        b_ag = burst(prefill_pair, reps)
        rec["prefill"] = dict(
            ms_per_step=ms_per_step, value_tops=ops / (ms_per_step * 1e-3) / 1e12,
            kernels={
                "requant_w_nvfp4_int8": dict(us_burst=b_w * 1e6, gbs=bytes_w / b_w / 1e9,
                                             frac_hbm=bytes_w / b_w / 1e9 / PEAK_HBM_GBS),
                "requant_a_int8": dict(us_burst=b_a * 1e6, gbs=bytes_a / b_a / 1e9,
                                       frac_hbm=bytes_a / b_a / 1e9 / PEAK_HBM_GBS),
                "int8_gemm_blockscaled": dict(us_in_step_mean=t_g.mean() * 1e6,
                                              us_in_step_median=float(np.median(t_g)) * 1e6,
                                              us_in_step_min=t_g.min() * 1e6,
                                              us_burst=b_g * 1e6, tops=gemm_tops,
                                              frac_int8=gemm_tops / PEAK_INT8_TOPS),
                "requant_a_plus_gemm": dict(us_burst=b_ag * 1e6, tops=ops / b_ag / 1e12),
            },
            buffer_sets=nsets)
        # the bursts reused the sets: recompute the output checked below
        step(sets[(args.steps - 1) % nsets])
        torch.cuda.synchronize()
        # parity of the timed outputs (last set used), sampled rows against the oracle
        s = sets[(args.steps - 1) % nsets]
        rows = np.array([0, 1, 777, M - 1])
        ow, osw = oracle.requant_w(packed, e4m3, proj.scale2)
        oa, osa = oracle.requant_a(a_bits[rows])
        y, t = oracle.gemm_ref(oa, ow, osa, osw)
        from oracle.compare import check_bf16
        res = check_bf16(s["out"][torch.as_tensor(rows, device=dev)].cpu().numpy().view(np.uint16), y, t, K)
        rec["prefill"]["parity_sampled_rows"] = dict(rows=len(rows), ok=res.ok, failures=res.failures)

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

    # ------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.no_cpu_baseline and args.only in ("all", "prefill"):
        cores = oracle.max_threads()
        t0 = time.perf_counter()
        ow, osw = oracle.requant_w(packed, e4m3, proj.scale2)
        t_rw = time.perf_counter() - t0
        t0 = time.perf_counter()
        oa, osa = oracle.requant_a(a_bits)
        t_ra = time.perf_counter() - t0
        rows_done, t_rows = 0, 0.0
        budget = max(1.0, args.cpu_seconds - t_rw - t_ra)
        chunk = max(1, cores)
        while t_rows < budget and rows_done < M:
            r = np.arange(rows_done, min(M, rows_done + chunk))
            t0 = time.perf_counter()
            oracle.gemm_ref(oa[r], ow, osa[r], osw)
            t_rows += time.perf_counter() - t0
            rows_done += len(r)
        t_full = t_rw + t_ra + t_rows * M / rows_done
        cpu = dict(value=2.0 * M * N * K / t_full / 1e12, unit="TOPS", cores=cores, kind="oracle",
                   sample=(f"full weight and activation requant ({t_rw:.2f} s + {t_ra:.2f} s), "
                           f"GEMM reference on {rows_done} of {M} rows ({t_rows:.2f} s) "
                           f"extrapolated linearly to all rows"),
                   seconds_extrapolated=t_full)
        # the same oracle on one thread: 256 weight rows, 64 activation rows and 16
        # GEMM rows, each extrapolated linearly to the whole workload
        oracle.set_threads(1)
        try:
            t0 = time.perf_counter()
            oracle.requant_w(packed[:256], e4m3[:256], proj.scale2)
            t1_w = (time.perf_counter() - t0) * N / 256
            t0 = time.perf_counter()
            oracle.requant_a(a_bits[:64])
            t1_a = (time.perf_counter() - t0) * M / 64
            t0 = time.perf_counter()
            oracle.gemm_ref(oa[:16], ow, osa[:16], osw)
            t1_g = (time.perf_counter() - t0) * M / 16
        finally:
            oracle.set_threads(cores)
        t1 = t1_w + t1_a + t1_g
        cpu["single_thread"] = dict(value=2.0 * M * N * K / t1 / 1e12, unit="TOPS", cores=1,
                                    sample="weight requant on 256 of N rows, activation requant on 64 of M "
                                           "rows, GEMM reference on 16 of M rows, each extrapolated linearly",
                                    seconds_extrapolated=t1)

    pre = rec.get("prefill")
    line = {
        "metric": METRIC,
        "value": pre["value_tops"] if pre else None,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"] if pre else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"prefill attention projection M={M} N={N} K={K} "
                               "(A ~ N(0,1) BF16, NVFP4 W scales 2^U{-4..2}, scale2 = fl32(1/448))",
                   "m": M, "n": N, "k": K,
                   "step": "requant_w_nvfp4_int8 + requant_a_int8 + int8_gemm_blockscaled"},
    }
    if pre:
        g = pre["kernels"]["int8_gemm_blockscaled"]
        line["roofline"] = {"bound": "mfma", "achieved": g["tops"], "peak": PEAK_INT8_TOPS,
                            "unit": "TOPS", "frac": g["tops"] / PEAK_INT8_TOPS,
                            "traffic": _traffic("gemm_kernel", ["gemm.hip", "bsr_internal.h"], None),
                            "kernel": "gemm_kernel (int8_gemm_blockscaled, m > 16)"}
        # The same kernel against the vector ALU, which bounds it: the exact
        # per-block FP32 rescale is one int32 -> FP32 conversion and one FMA per
        # output and 32-wide K block; peak = 256 CUs x 4 SIMDs x 16 lanes x
        # 2.4 GHz non-packed FP32 lane operations.
        alu_ops = 2.0 * M * N * (K // 32)
        alu = alu_ops / (g["us_in_step_mean"] * 1e-6) / 1e12
        line["roofline_alu"] = {"bound": "alu", "achieved": alu, "peak": PEAK_VALU_TOPS,
                                "unit": "T lane-ops/s", "frac": alu / PEAK_VALU_TOPS,
                                "work": "int32->FP32 conversion + FMA per output and K block"}
        line["kernels"] = pre["kernels"]
        line["parity"] = pre["parity_sampled_rows"]
    if cpu:
        line["cpu_baseline"] = cpu
    if "decode" in rec:
        line["decode"] = rec["decode"]
    if "silu" in rec:
        line["silu_mul_requant"] = rec["silu"]
    if "layouts" in rec:
        line["activation_layouts"] = rec["layouts"]
    if "copy_context" in rec:
        line["copy_context"] = rec["copy_context"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
