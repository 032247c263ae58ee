#!/usr/bin/env python3
"""Throughput of the ARL2 hybrid attention layer on one MI355X.

A step is one frame of the streaming loop of the Wan-1.3B-shaped layer
(1 video x 12 heads x 128, T = 1560 tokens per frame, bf16 activations, fp32
state): 4 denoising reads and the clean pass (its read plus the state commit),
i.e. every step of the hot path: feature maps, intra-frame softmax, inter-frame
read, combine, state commit. Inputs are seeded synthetic tensors resident in
HBM before timing starts (a pool of frames is cycled); the state carries over
from frame to frame. Each frame's calls are launched on the stream as the layer
driver issues them (replays of a HIP graph of the same launches are timed
beside, or instead with --graph; on this stack both run at about the same rate).

Printed (one JSON line): frames/s (value) and tokens/s, the roofline of the
dominant kernel (the fused read: intra-frame attention plus the inter-frame
read, bf16 MFMA, five launches per frame) measured with HIP events on the
launch stream over the same cycling inputs as the step, per-kernel times, the fp64 CPU oracle timed on this host on
a bounded sample, and the flatness of per-frame time and memory over a long
rollout beside the full-KV-cache softmax comparator.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]
    python bench.py --workload batched_streams   # 8 videos (8 x 12 heads)
    python bench.py --workload large_model       # 40 heads
    python bench.py --sweep-read                 # the fused read across shapes

The two other workloads time the same step at their shapes (without the
traffic counters, the rollout and the oracle baseline, which are taken on the
one-layer shape).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_MFMA = 2.5e15        # dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12              # HBM3E, B/s
COMMIT_BYTES_PER_HEAD = None   # filled from the shape: 2*T*D*2 + 4*T + 2*D*D*4


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed frames")
    ap.add_argument("--warmup", type=int, default=20, help="untimed frames")
    ap.add_argument("--workload", default="wan13b_layer",
                    choices=["wan13b_layer", "batched_streams", "large_model"],
                    help="the one-layer shape (the reported metric), 8 videos of it, or 40 heads")
    ap.add_argument("--pool", type=int, default=None,
                    help="distinct resident input frames (even; one graph covers them all; "
                         "default: enough frames for >= 512 MB of inputs, at least 2)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of the pool's frames instead of launching "
                         "each frame's calls on the stream")
    ap.add_argument("--no-graph-compare", action="store_true",
                    help="skip the extra graph-replay timing reported beside the value")
    ap.add_argument("--kernel-iters", type=int, default=50)
    ap.add_argument("--rollout-frames", type=int, default=240)
    ap.add_argument("--skip-rollout", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="instead of the step: read two rocprofv3 --pmc --output-format csv runs "
                         "of this script (FETCH_SIZE, then WRITE_SIZE), scale them by the copy "
                         "calibration's known bytes, write profiles/traffic.json and print a "
                         "table (no GPU needed)")
    ap.add_argument("--sweep-read", action="store_true",
                    help="instead of the step: time the fused read (arl2_read_prepared) across "
                         "frame lengths, heads and videos, one JSON line per shape")
    return ap.parse_args()


# the sources the frame-level kernels are compiled from
FRAME_KERNEL_SOURCES = ("kernels_mfma.hip", "mfma_common.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hybrid_linear_memory_amd", "csrc")
    for name in FRAME_KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(kernel)
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return ent.get("bytes_per_launch")


class Bench:
    def __init__(self, args):
        import torch

        from hybrid_linear_memory_amd import arl2, synth
        from hybrid_linear_memory_amd.layer import Arl2Layer

        self.torch, self.arl2, self.synth = torch, arl2, synth
        self.args = args
        self.w = next(x for x in synth.WORKLOADS.values() if x.name == args.workload)
        w = self.w
        if args.pool is None:
            per_frame = w.passes * 3 * w.B * w.H * w.T * w.D * 2
            args.pool = max(2, -(-(512 << 20) // per_frame))
            args.pool += args.pool % 2
        self.shape = arl2.Shape(w.B, w.H, w.T, w.D, arl2.BF16)
        self.stream = torch.cuda.current_stream()
        bf = torch.bfloat16

        def dev(x, dt=bf):
            return torch.from_numpy(x).to("cuda").to(dt).contiguous()

        self.dev = dev
        phis = synth.phi_maps(w)
        self.layer = Arl2Layer(self.shape, *[dev(p) for p in phis])
        # pool of resident frames: passes[p] = (q, k, v), plus gates
        self.pool = []
        for f in range(args.pool):
            passes = [tuple(dev(x) for x in synth.qkv(w, f, p)) for p in range(w.passes)]
            beta, alpha = synth.gates(w, f)
            self.pool.append((passes, dev(beta, torch.float32), dev(alpha, torch.float32)))
        self.out = [self.layer.new_output() for _ in range(w.passes)]
        torch.cuda.synchronize()

    def frame(self, i):
        passes, beta, alpha = self.pool[i % len(self.pool)]
        L = self.layer
        for p in range(self.w.n_denoise):
            L.read(*passes[p], o=self.out[p])
        L.clean_pass(*passes[-1], beta, alpha, o=self.out[-1])

    def run_frames(self, n_frames, start=0):
        for i in range(n_frames):
            self.frame(start + i)

    def make_graph(self):
        """One graph over all pool frames (an even number: the state and the
        prepared map ping-pong between two buffers each, so the graph returns
        them to the buffers it started from)."""
        torch = self.torch
        assert len(self.pool) % 2 == 0
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.layer.seq.restore(self.layer.frame)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for i in range(len(self.pool)):
                    self.frame(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        return g

    def timed(self, steps, warmup, use_graph):
        torch = self.torch
        if use_graph:
            g = self.make_graph()
            per = len(self.pool)
            n_rep = (steps + per - 1) // per
            for i in range(max(1, (warmup + per - 1) // per)):
                g.replay()
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            w0 = time.perf_counter()
            for i in range(n_rep):
                g.replay()
            t1.record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - w0
            frames = per * n_rep
        else:
            self.run_frames(warmup)
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            w0 = time.perf_counter()
            self.run_frames(steps)
            t1.record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - w0
            frames = steps
        gpu_ms = t0.elapsed_time(t1)
        self.last_host_s = wall
        return frames, max(gpu_ms / 1e3, wall), gpu_ms / 1e3

    def kernel_times(self, iters):
        """Average launch duration of each kernel of the path, from HIP events
        around back-to-back launches on the launch stream. As in the step,
        consecutive launches take different resident input sets (the pool's
        frames x passes), so a launch does not find its inputs in cache from
        the launch before."""
        torch, arl2, sh = self.torch, self.arl2, self.shape
        sets = [(q, k, v, beta, alpha) for (passes, beta, alpha) in self.pool
                for (q, k, v) in passes]
        n = len(sets)
        L = self.layer
        tmp = [L.new_output() for _ in range(3)]
        S_next = torch.empty_like(L.S)
        ws = arl2.alloc_workspace(sh, arl2.OP_STATE_COMMIT)
        # mapped (K', V') of every input set, for the commit from given K', V'
        mapped = []
        for (_, k, v, _, _) in sets:
            kp, vp = L.new_output(), L.new_output()
            arl2.feature_map(sh, k, L.phi[1], kp, True)
            arl2.feature_map(sh, v, L.phi[2], vp, False)
            mapped.append((kp, vp))
        rws = arl2.alloc_workspace(sh, arl2.OP_READ)
        cws = arl2.alloc_workspace(sh, arl2.OP_COMMIT)
        M = arl2.alloc_prepared(sh)
        arl2.read_prepare(sh, L.phi[0], L.S, M)
        cases = {
            "intra_attn": lambda i: arl2.intra_attn(sh, *sets[i % n][:3], tmp[0]),
            "read": lambda i: arl2.read(sh, *sets[i % n][:3], L.phi[0], L.S, tmp[0], ws=rws),
            "read_prepare": lambda i: arl2.read_prepare(sh, L.phi[0], L.S, M),
            "read_prepared": lambda i: arl2.read_prepared(sh, *sets[i % n][:3], M, tmp[0],
                                                          ws=rws),
            "feature_map": lambda i: arl2.feature_map(sh, sets[i % n][0], L.phi[0], tmp[0],
                                                      False),
            # from mapped K', V' (this entry point is not on the step)
            "state_commit": lambda i: arl2.state_commit(sh, *mapped[i % n], sets[i % n][3],
                                                        sets[i % n][4], L.S, S_next, ws),
            "commit": lambda i: arl2.commit(sh, sets[i % n][1], sets[i % n][2], L.phi[1],
                                            L.phi[2], sets[i % n][3], sets[i % n][4], L.S,
                                            S_next, cws),
        }
        res = {}
        for name, fn in cases.items():
            for i in range(n):
                fn(i)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(iters):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) / iters * 1e3   # microseconds
        return res

    def copy_calibration(self, nbytes=1 << 30):
        """Two device kernels of known traffic, so that rocprofv3 counter runs
        of this script can scale FETCH_SIZE / WRITE_SIZE against known bytes
        (the copy) and check the scale on a kernel of another shape (the add:
        two inputs read, one output written)."""
        torch = self.torch
        a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        a2 = torch.empty_like(a).fill_(2.0)
        b = torch.empty_like(a)
        torch.add(a[:1024], a2[:1024], out=b[:1024])      # the add's kernel loaded
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        b.copy_(a)
        ev[1].record()
        torch.add(a, a2, out=b)
        ev[2].record()
        torch.cuda.synchronize()
        ms_copy, ms_add = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
        del a, a2, b
        return {"bytes_read": nbytes, "bytes_written": nbytes,
                "GBps": 2 * nbytes / (ms_copy / 1e3) / 1e9,
                "add_bytes_read": 2 * nbytes, "add_bytes_written": nbytes,
                "add_GBps": 3 * nbytes / (ms_add / 1e3) / 1e9}

    def rollout_flatness(self, n_frames, warm_frames=120):
        """Per-frame time and device memory over a long rollout of the layer,
        beside the full-KV-cache softmax comparator at the same shapes.

        The layer first runs warm_frames frames, then resets its state (S = 0)
        and runs the n_frames measured frames right after them, with no
        synchronisation in between, so that the measured frames meet the
        clocks and the launch queue of the steady frame loop (the frames
        straight after the kernel timings otherwise run a few percent slow and
        drift down). Reported: the mean of every 20-frame window, the slope of
        a linear fit over all measured frames, and flat = |slope| x n_frames
        below 5% of the mean."""
        import numpy as np
        torch, arl2, sh, w = self.torch, self.arl2, self.shape, self.w
        L = self.layer
        torch.cuda.synchronize()
        for f in range(warm_frames):
            self.frame(f)
        L.reset()
        mem0 = torch.cuda.memory_allocated()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_frames + 1)]
        ev[0].record()
        for f in range(n_frames):
            self.frame(f)
            ev[f + 1].record()
        torch.cuda.synchronize()
        mem1 = torch.cuda.memory_allocated()
        t_arl2 = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n_frames)])
        # comparator: the cache grows by one frame of K and V per clean pass;
        # its buffers hold all n_frames frames from the start (allocated bytes
        # measured), each frame attends over the frames cached so far
        cap = n_frames * w.T
        m_before = torch.cuda.memory_allocated()
        kc = torch.empty((w.B, w.H, cap, w.D), dtype=torch.bfloat16, device="cuda")
        vc = torch.empty_like(kc)
        cache_alloc = torch.cuda.memory_allocated() - m_before
        o = L.new_output()
        ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(n_frames + 1)]
        ev2[0].record()
        for f in range(n_frames):
            passes, _, _ = self.pool[f % len(self.pool)]
            sl = slice(f * w.T, (f + 1) * w.T)
            for (q, k, v) in passes:
                kc[:, :, sl].copy_(k)
                vc[:, :, sl].copy_(v)
                arl2.fullkv_attn(sh, q, kc, vc, (f + 1) * w.T, o)
            ev2[f + 1].record()
        torch.cuda.synchronize()
        t_full = np.array([ev2[i].elapsed_time(ev2[i + 1]) for i in range(n_frames)])
        del kc, vc
        x = np.arange(n_frames)
        slope = float(np.polyfit(x, t_arl2, 1)[0]) if n_frames > 2 else 0.0
        slope_full = float(np.polyfit(x, t_full, 1)[0]) if n_frames > 2 else 0.0
        mean = float(t_arl2.mean())
        win = 20
        windows = [float(t_arl2[i:i + win].mean()) for i in range(0, n_frames, win)]
        return {
            "frames": n_frames,
            "warmup_frames": warm_frames,
            "arl2_ms_per_frame_mean": mean,
            "arl2_ms_first_last": [float(t_arl2[0]), float(t_arl2[-1])],
            "arl2_ms_per_frame_window_means": windows,
            "arl2_slope_ms_per_frame": slope,
            "arl2_flat": abs(slope * n_frames) < 0.05 * mean,
            "arl2_state_bytes": 2 * w.B * w.H * w.D * w.D * 4,
            "arl2_device_mem_delta_bytes": int(mem1 - mem0),
            "fullkv_ms_first_last": [float(t_full[0]), float(t_full[-1])],
            "fullkv_slope_ms_per_frame": slope_full,
            "fullkv_cache_bytes_last": 2 * cap * w.D * 2 * w.B * w.H,
            "fullkv_cache_bytes_allocated": int(cache_alloc),
            "fullkv_total_ms": float(t_full.sum()),
            "arl2_total_ms": float(t_arl2.sum()),
            "speedup_total": float(t_full.sum() / t_arl2.sum()),
        }


SWEEP_SHAPES = [(1, 12, 1560), (1, 12, 3600), (1, 12, 6240), (2, 12, 1560), (4, 12, 1560),
                (8, 12, 1560), (1, 40, 1560), (1, 4, 4096), (1, 2, 8192)]


def sweep_read(base_iters: int):
    """The fused read (arl2_read_prepared, with a workspace so that the shapes
    that take the split-key grid do) at d = 128 across (B, H, T): launches back
    to back on one stream over a pool of resident inputs of at least 512 MB
    (so that they come from HBM), each shape warmed up for as many launches as
    it times, timed with HIP events. Inputs follow the workloads' recipe (Q, K,
    V standard normal, keys L2-normalised row by row). Work per launch: 4 T^2 d
    (Q K^T and P V) plus 2 T d^2 (Q M) FLOP per head, against the dense bf16
    MFMA peak."""
    import torch

    from hybrid_linear_memory_amd import arl2
    for B, H, T in SWEEP_SHAPES:
        sh = arl2.Shape(B, H, T, 128, arl2.BF16)
        g = torch.Generator(device="cuda").manual_seed(0)
        n_sets = max(2, -(-(512 << 20) // (3 * B * H * T * 128 * 2)))

        def qkv():
            q, k, v = (torch.randn(B, H, T, 128, generator=g, device="cuda") for _ in range(3))
            k = k / k.norm(dim=-1, keepdim=True)
            return tuple(x.to(torch.bfloat16) for x in (q, k, v))

        sets = [qkv() for _ in range(n_sets)]
        M = arl2.alloc_prepared(sh)
        phi = (torch.randn(H, 128, 128, generator=g, device="cuda") * 128 ** -0.5).to(
            torch.bfloat16)
        arl2.read_prepare(sh, phi, torch.randn(B, H, 128, 128, generator=g, device="cuda") * 0.05,
                          M)
        o = torch.empty(B, H, T, 128, dtype=torch.bfloat16, device="cuda")
        ws = arl2.alloc_workspace(sh, arl2.OP_READ_PREPARED)
        split = arl2.workspace_bytes(sh, arl2.OP_READ_PREPARED) > 0
        iters = max(20, base_iters * 1560 * 12 // (T * H * B))
        for i in range(iters):
            arl2.read_prepared(sh, *sets[i % n_sets], M, o, ws=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            arl2.read_prepared(sh, *sets[i % n_sets], M, o, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / iters
        flop = B * H * (4.0 * T * T * 128 + 2.0 * T * 128 * 128)
        print(json.dumps({"B": B, "H": H, "T": T, "split_key_grid": split,
                          "query_blocks": B * H * (-(-T // 128)), "us": round(us, 2),
                          "tflops": round(flop / us / 1e6, 1),
                          "frac_of_bf16_peak": round(flop / (us * 1e-6) / PEAK_BF16_MFMA, 4)}),
              flush=True)
        del sets


def cpu_baseline(seconds: float):
    """The fp64 oracle, as it stands, on this host: whole frames of the same
    workload (4 reads + clean pass, all heads) until ~`seconds` of CPU time,
    at least 2 frames. Input generation is outside the timed part."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    from hybrid_linear_memory_amd import synth
    cores = len(os.sched_getaffinity(0))
    w = synth.WORKLOADS[1]
    phis = synth.phi_maps(w)
    with threadpool_limits(limits=cores):
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
        S = np.zeros((w.B, w.H, w.D, w.D))
        frames, busy = 0, 0.0
        est = None
        while frames < 2 or (busy < seconds and frames < w.frames):
            fr = synth.oracle_frame(w, frames)
            t0 = time.perf_counter()
            _, states = oracle.rollout([fr], *phis, S0=S)
            busy += time.perf_counter() - t0
            S = states[-1]
            frames += 1
            est = busy / frames
            if busy + est > 2.5 * seconds:
                break
    # beside it: one BLAS thread (one whole frame), the commit alone at all
    # cores (frames/s of the clean pass's state write), the tiny fp32 workload
    # end to end
    fr = synth.oracle_frame(w, 0)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.rollout([fr], *phis, S0=np.zeros((w.B, w.H, w.D, w.D)))
        one_thread = 1.0 / (time.perf_counter() - t0)
    with threadpool_limits(limits=cores):
        _, kc, vc = fr["passes"][-1]
        n_c, t0 = 0, time.perf_counter()
        while n_c < 3 or time.perf_counter() - t0 < 1.0:
            oracle.commit(kc, vc, phis[1], phis[2], fr["beta"], fr["alpha"],
                          np.zeros((w.B, w.H, w.D, w.D)))
            n_c += 1
        commit_only = n_c / (time.perf_counter() - t0)
        w0 = synth.WORKLOADS[0]
        frames0 = [synth.oracle_frame(w0, f) for f in range(w0.frames)]
        t0 = time.perf_counter()
        oracle.rollout(frames0, *synth.phi_maps(w0))
        tiny_s = time.perf_counter() - t0
    threads = max((n for _, n in blas if n), default=1)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": frames / busy,
        "unit": "frames/s",
        "cores": int(min(threads, cores)),
        "kind": "oracle",
        "sample": f"{frames} whole frames of the 1x12x128, T=1560 layer (4 reads + clean pass "
                  f"each), fp64 numpy, {busy:.1f} s",
        "tokens_per_s": frames * w.T / busy,
        "one_thread_frames_per_s": one_thread,
        "commit_only_frames_per_s": commit_only,
        "tiny_fp32_rollout_s": tiny_s,
        "cpu_model": cpu_model,
        "blas": blas,
    }


CALIB_BYTES = 1 << 30


def _short_kernel(name: str) -> str:
    """rocprofv3 kernel name -> the short name used in profiles/traffic.json."""
    import re
    if name.startswith("_Z"):
        # mangled (rocprofv3 leaves names with __bf16 parameters mangled):
        # <len><name>[I<template args>E]..., bool arguments as Lb0E / Lb1E,
        # int arguments as Li<n>E
        i = name.find("N", 2) + 1 if name.startswith("_ZN") else 2
        ident = ""
        while i < len(name) and name[i].isdigit():
            j = i
            while name[j].isdigit():
                j += 1
            n = int(name[i:j])
            ident, i = name[j:j + n], j + n
        m = re.match(r"I((?:L[bi]\d+E)+)E", name[i:])
        if ident:
            args = ["true" if a == "b1" else "false" if a == "b0" else a[1:]
                    for a in re.findall(r"L([bi]\d+)E", m.group(1) if m else "")]
            name = f"{ident}<{', '.join(args)}>(" if args else f"{ident}("
    m = re.search(r"(\w+_k)(<([^()]*)>)?\(", name)
    if m:
        base, targs = m.group(1), (m.group(3) or "")
        args = [a.strip() for a in targs.split(",")] if targs else []
        if base == "attn_mfma_k" and args:
            return f"attn_mfma_k<{args[0]}>" + (" (LSE)" if len(args) > 1 and args[1] == "true"
                                                 else "")
        if base == "rowmap_mfma_k" and args:
            return {"0": "rowmap_mfma_k<MAP_PHI> (feature map)",
                    "1": "rowmap_mfma_k<MAP_STATE>"}.get(args[0], name)
        return base
    if "copyBuffer" in name:
        return "copyBuffer"
    if "elementwise" in name and "add" in name.lower():
        return "elementwise_add"
    return name[:60]


def _read_counter_csv(d: str, counter: str):
    """(short kernel name, grid size, value) per dispatch from the
    counter_collection csv files under d."""
    import csv
    rows = []
    for dirpath, _, files in os.walk(d):
        for fn in files:
            if not fn.endswith("counter_collection.csv"):
                continue
            with open(os.path.join(dirpath, fn), newline="") as f:
                for r in csv.DictReader(f):
                    low = {k.lower(): v for k, v in r.items()}
                    if low.get("counter_name") != counter:
                        continue
                    rows.append((_short_kernel(low["kernel_name"]), int(low["grid_size"]),
                                 float(low["counter_value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {d}")
    return rows


def traffic_from(fetch_dir: str, write_dir: str):
    """HBM bytes per launch of each kernel from a FETCH_SIZE run and a
    WRITE_SIZE run (KiB per dispatch), scaled so that the calibration copy
    reads and writes its known 1 GiB; the calibration add (2 GiB read, 1 GiB
    written) checks the scale on a kernel of another shape. Per kernel: the
    median dispatch of its largest grid. Writes profiles/traffic.json."""
    import re
    import statistics
    fetch = _read_counter_csv(fetch_dir, "FETCH_SIZE")
    write = _read_counter_csv(write_dir, "WRITE_SIZE")

    def largest(rows, kernel):
        sel = [(g, v) for k, g, v in rows if k == kernel]
        if not sel:
            return None, None
        gmax = max(g for g, _ in sel)
        return gmax, statistics.median(v for g, v in sel if g == gmax)

    _, f_copy = largest(fetch, "copyBuffer")
    _, w_copy = largest(write, "copyBuffer")
    ff = CALIB_BYTES / (f_copy * 1024.0)
    fw = CALIB_BYTES / (w_copy * 1024.0)
    _, f_add = largest(fetch, "elementwise_add")
    _, w_add = largest(write, "elementwise_add")
    check = None
    if f_add and w_add:
        check = {"add_read_ratio": f_add * 1024.0 * ff / (2 * CALIB_BYTES),
                 "add_write_ratio": w_add * 1024.0 * fw / CALIB_BYTES}
    src_hash = kernel_source_hash()
    out = {}
    names = sorted({k for k, _, _ in fetch} & {k for k, _, _ in write})
    for k in names:
        if k in ("copyBuffer", "elementwise_add") or not re.match(r"^\w+_k\b", k):
            continue
        g, fv = largest(fetch, k)
        g2, wv = largest(write, k)
        if g != g2:
            continue
        out[k] = {"bytes_per_launch": fv * 1024.0 * ff + wv * 1024.0 * fw, "grid": g,
                  "fetch_bytes": fv * 1024.0 * ff, "write_bytes": wv * 1024.0 * fw,
                  "source_hash": src_hash,
                  "note": f"FETCH_SIZE*{ff:.3f} + WRITE_SIZE*{fw:.3f} (KiB x 1024), median "
                          "dispatch of the largest grid"}
    out["_calibration"] = {"fetch_scale": ff, "write_scale": fw, "add_check": check,
                           "copy_bytes": CALIB_BYTES}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(f"scales: FETCH_SIZE x {ff:.3f}, WRITE_SIZE x {fw:.3f}; add check {check}")
    print("| kernel | grid | read MB | written MB | total MB |")
    print("|---|---|---|---|---|")
    for k, e in sorted(out.items()):
        if k.startswith("_"):
            continue
        print(f"| {k} | {e['grid']} | {e['fetch_bytes'] / 1e6:.2f} | {e['write_bytes'] / 1e6:.2f} "
              f"| {e['bytes_per_launch'] / 1e6:.2f} |")


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the layer shards "
              "by (video, head) with no exchange inside the step, and this program measures "
              "the one-GPU share.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.sweep_read:
        sweep_read(4 * args.steps)
        return
    print("[bench] building the pool of input frames", file=sys.stderr, flush=True)
    b = Bench(args)
    print(f"[bench] pool of {args.pool} frames resident", file=sys.stderr, flush=True)
    w = b.w
    calib = b.copy_calibration()
    print("[bench] timing frames", file=sys.stderr, flush=True)
    frames, secs, gpu_secs = b.timed(args.steps, args.warmup, use_graph=args.graph)
    host_secs = b.last_host_s
    fps = w.B * frames / secs
    other = None
    if not args.no_graph_compare:
        of, os_, _ = b.timed(max(40, args.steps // 2), 8, use_graph=not args.graph)
        other = w.B * of / os_
    print("[bench] timing kernels", file=sys.stderr, flush=True)
    kt = b.kernel_times(args.kernel_iters)
    # The dominant kernel: the fused read (attn_mfma_k<true>), five launches per
    # frame. Algorithmic flops per launch: Q K^T and P V (2 x 2 T^2 D per head)
    # plus the inter-frame read Q M (2 T D^2 per head).
    flops_intra = 4.0 * w.T * w.T * w.D * w.B * w.H
    flops = flops_intra + 2.0 * w.T * w.D * w.D * w.B * w.H
    attn_s = kt["read_prepared"] * 1e-6
    achieved = flops / attn_s
    src_hash = kernel_source_hash()
    traffic = load_traffic("attn_mfma_k<true>", src_hash)
    # the state write's algorithmic bytes: K and V (bf16; K', V' for the
    # commit from mapped inputs), beta (fp32), S_prev read and S_next written
    # (fp32); the commit from raw K, V also reads the two feature maps per head
    commit_bytes = w.B * w.H * (2 * w.T * w.D * 2 + 4 * w.T + 2 * w.D * w.D * 4)
    commit_raw_bytes = commit_bytes + w.H * 2 * w.D * w.D * 2
    kernels = {
        "intra_attn_us": kt["intra_attn"],
        "intra_attn_tflops": flops_intra / (kt["intra_attn"] * 1e-6) / 1e12,
        "read_us": kt["read"],
        "read_prepare_us": kt["read_prepare"],
        "read_prepared_us": kt["read_prepared"],
        "feature_map_us": kt["feature_map"],
        # the commit on the step: commit_col_k (arl2_commit; the clean pass
        # runs the same code on the compute units its read leaves idle)
        "commit_us": kt["commit"],
        "commit_kernel": "commit_col_k",
        "commit_hbm_frac": commit_raw_bytes / (kt["commit"] * 1e-6) / PEAK_HBM,
        "commit_algorithmic_bytes": commit_raw_bytes,
        # arl2_state_commit from mapped K', V' (commit_mfma_k + commit_reduce_k;
        # not on the step)
        "state_commit_us": kt["state_commit"],
        "state_commit_kernels": "commit_mfma_k+commit_reduce_k",
        "state_commit_hbm_frac": commit_bytes / (kt["state_commit"] * 1e-6) / PEAK_HBM,
        "state_commit_algorithmic_bytes": commit_bytes,
        "copy_calibration": calib,
    }
    one_layer = args.workload == "wan13b_layer"
    if not one_layer:
        # the traffic counters, the flatness rollout and the oracle baseline are
        # taken on the one-layer shape only
        traffic, args.skip_rollout, args.skip_cpu = None, True, True
    flat = None
    if not args.skip_rollout:
        print("[bench] rollout flatness", file=sys.stderr, flush=True)
        flat = b.rollout_flatness(args.rollout_frames)
    cpu = None
    if not args.skip_cpu:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.cpu_seconds)
    res = {
        "metric": ("ARL2 layer frames/sec (12x128 heads, 1560 tok/frame)" if one_layer else
                   f"ARL2 layer frames/sec ({w.B} video{'s' if w.B > 1 else ''} x {w.H}x{w.D} "
                   f"heads, {w.T} tok/frame)"),
        "value": fps,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": frames,
        "warmup": args.warmup,
        "ms_per_step": secs / frames * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.B} video{'s' if w.B > 1 else ''} x {w.H} heads "
                               f"x d{w.D}, T={w.T} tokens/frame, {w.n_denoise} denoising reads + "
                               "clean pass (read + state commit) per frame, bf16 activations, "
                               "fp32 state",
                   "B": w.B, "H": w.H, "D": w.D, "T": w.T, "passes_per_frame": w.passes,
                   "hip_graph": args.graph},
        "tokens_per_s": fps * w.T,
        # the step's two clocks: GPU events around the timed frames, and the
        # host's wall time to issue them (value uses the larger)
        "gpu_ms_per_step": gpu_secs / frames * 1e3,
        "host_ms_per_step": host_secs / frames * 1e3,
        ("frames_per_s_stream" if args.graph else "frames_per_s_graph"): other,
        "roofline": {"bound": "mfma",
                     "kernel": "attn_mfma_k<true> (fused read: intra-frame softmax + Q M)",
                     "achieved": achieved / 1e12, "peak": PEAK_BF16_MFMA / 1e12,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_MFMA,
                     "traffic": traffic, "flop_per_launch": flops,
                     "avg_launch_us": kt["read_prepared"]},
        "kernels": kernels,
        "flatness": flat,
        "cpu_baseline": cpu,
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
