"""Benchmark of the attention hot path on one MI355X.

One step = the whole path on one batch of the 5 s 1344x768 video workload (latent grid
31 x 48 x 84 = 124,992 tokens, 48 heads, head_dim 128, smooth-field q/k, N(0,1) v, bf16):
  qk_norm_rope_pool (norm+RoPE, pooling q' and k' for the selection in the same pass) -> dense_fwd
  -> subblock_select_pooled (sparsity 0.75) -> block_sparse_fwd.
Inputs are resident in HBM before the timed region; outputs and workspaces are preallocated.
After the timed steps, norm+RoPE alone and the selection with its own pooling pass (the
stand-alone calls) are timed on the same inputs, and their kept sets compared with the step's.

Printed JSON line: value = attention TFLOP/s of the step (dense 4*B*H*N^2*D plus block-sparse
4*B*H*nB*keep*64^2*D flops, divided by the whole step's time, norm+RoPE and selection included).
Per-kernel times come from HIP events recorded on the launch stream between the calls of every
timed step; `roofline` describes the dense kernel (the dominant one) against the bf16 MFMA peak.
`cpu_baseline` times every stage of the float64 oracle (norm+RoPE, selection, dense and sparse
attention) on bounded samples of the same workload on the host cores, each extrapolated to the
whole step and labelled so.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn TFLOP/s (% MFMA peak) dense+SubBlock 0.75; QK-norm+RoPE HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--config", type=int, default=3,
                   help="workload id: 1 tiny, 2 one frame, 3 the 5 s video (default), 4 the 10 s video, 5 the 15 s video")
    p.add_argument("--sparsity", type=float, default=0.75)
    p.add_argument("--group-stride", type=int, default=0,
                   help="query-block group stride of the sparse kernels (0: one frame of blocks when frames "
                        "are whole blocks, else 1)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=16.0, help="target CPU time of the oracle samples")
    p.add_argument("--no-extra", action="store_true",
                   help="skip everything outside the step: flushed norm+RoPE, block ops, threshold mode, fp8, "
                        "the 10 s and 15 s workloads and the context rates")
    p.add_argument("--no-clock", action="store_true",
                   help="do not read the GFX clock with amd-smi during the timed steps (for profiled runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first copy 1 GiB once, so that memory counters of a known-size copy sit in the same trace")
    return p.parse_args()


def measured_traffic(kernel_prefix: str):
    """Bytes per launch of a kernel from the committed PMC summary, or None when the kernel's
    source has changed since the counters were taken (sha256 prefix recorded in the summary)."""
    import hashlib
    summary = os.path.join(ROOT, "profiles", "pmc_traffic_video5s.txt")
    src = os.path.join(ROOT, "video_diffusion_transformer_qk_amd", "csrc", "attention.hip")
    try:
        lines = open(summary).read().splitlines()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    recorded = [l.split(":", 1)[1].strip() for l in lines if l.startswith("attention_source_sha256:")]
    if not recorded or recorded[0] != sha:
        return None
    for l in lines:
        if l.startswith(kernel_prefix):
            return float(l.split("|")[3].strip())
    return None


def measured_traffic_range():
    """The dense kernel's scaled traffic over every PMC pass recorded in the summary's header (its
    L2 hit rate, and so its FETCH_SIZE, varies between passes), or None."""
    summary = os.path.join(ROOT, "profiles", "pmc_traffic_video5s.txt")
    try:
        text = open(summary).read()
    except OSError:
        return None
    import re
    m = re.search(r"passes so far read ([0-9, and\n#]+?) KiB", text)
    w = [l for l in text.splitlines() if l.startswith("attn_fwd_kernel<")]
    if not m or not w:
        return None
    fetch = [float(x) for x in re.findall(r"[0-9]+", m.group(1))]
    write_kib = float(w[0].split("|")[2])
    return [(min(fetch) * 2.0 + write_kib) * 1024, (max(fetch) * 2.0 + write_kib) * 1024]


def provenance(cfg):
    """What produced this line: library and runtime versions, the device, the first 16 hex digits
    of each library source's sha256 (the tree is copied without version-control metadata) and the
    input recipe."""
    import hashlib
    import video_diffusion_transformer_qk_amd as h3
    from inputs import seed_for
    csrc = os.path.join(ROOT, "video_diffusion_transformer_qk_amd", "csrc")
    srcs = {}
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            srcs[f] = hashlib.sha256(open(os.path.join(csrc, f), "rb").read()).hexdigest()[:16]
    return {"library": h3.version(), "torch": torch.__version__, "hip": torch.version.hip,
            "device": torch.cuda.get_device_name(0), "sources_sha256": srcs,
            "inputs": {"field": cfg.field, "seeds": {t: seed_for(cfg.id, t) for t in ("q", "k", "v", "wq", "wk")}}}


class ClockSampler:
    """The GFX clock (MHz, mean over the XCDs) read with `amd-smi metric --clock --json` from a
    thread while the timed steps run. Reading clocks changes nothing on the device; the result is
    None when amd-smi is missing or its output cannot be read."""

    def __init__(self, period_s: float = 0.25, enabled: bool = True):
        import shutil
        import threading
        self.exe = shutil.which("amd-smi") if enabled else None
        self.cmd = None
        if self.exe:
            # a Python tool is started with this interpreter directly: its launcher line would
            # otherwise have a helper process exec the interpreter
            try:
                with open(self.exe, "rb") as f:
                    first = f.readline()
            except OSError:
                first = b""
            self.cmd = [sys.executable, self.exe] if first.startswith(b"#!") and b"python" in first else [self.exe]
        self.period = period_s
        self.samples = []
        self.done = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True) if self.exe else None

    def _read(self):
        import subprocess
        r = subprocess.run(self.cmd + ["metric", "--clock", "--json"], capture_output=True, text=True, timeout=10)
        data = json.loads(r.stdout)
        clk = data["gpu_data"][0]["clock"]
        vals = [v["clk"]["value"] for key, v in clk.items() if key.startswith("gfx_") and isinstance(v, dict)]
        vals = [float(x) for x in vals if isinstance(x, (int, float))]
        return sum(vals) / len(vals) if vals else None

    def _run(self):
        while not self.done.is_set():
            try:
                v = self._read()
                if v is not None:
                    self.samples.append(v)
            except Exception:  # noqa: BLE001 - a context figure only
                return
            self.done.wait(self.period)

    def start(self):
        if self.thread is not None:
            self.thread.start()
        return self

    def stop(self):
        if self.thread is None:
            return None
        self.done.set()
        self.thread.join(timeout=15)
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1], "samples": len(v),
                "source": "amd-smi metric --clock, mean of the gfx_* clocks, sampled during the timed steps"}


def flush_caches(buf: torch.Tensor):
    buf.add_(1)  # rewrites 512 MB: evicts the 256 MB MALL and every L2


def elapsed_ms(a, b):
    return a.elapsed_time(b)


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return int(os.cpu_count() or 1)


def cpu_baseline(q_in, k_in, wq, wk, q, k, v, cfg, sparsity, target_s):
    """The float64 oracle timed stage by stage on the host, on bounded samples of the step's own
    workload, each extrapolated to the whole workload (labelled as extrapolated):
      norm+RoPE   the first frames of the grid, every head (numpy ufuncs: one core);
      select      block means, block scores and top-k of a few whole heads (scores by BLAS);
      dense       sampled query blocks of several heads against all keys (BLAS);
      sparse      sampled query blocks over their oracle kept sets (BLAS).
    value = the step's attention flops (dense + kept sparse) / the extrapolated oracle step time,
    the same unit as the GPU line. Inputs: the raw q, k and weights (norm+RoPE) and the normed q, k
    and v that the other stages consume."""
    import oracle
    f64 = lambda t: t.detach().cpu().to(torch.float64).numpy()
    b, n, hd, d = q.shape
    nb = (n + 63) // 64
    keep = oracle.keep_count(nb, sparsity)
    rng = np.random.default_rng(0)
    stages = {}
    share = {"norm_rope": 0.15, "select": 0.25, "dense": 0.4, "sparse": 0.2}

    # norm+RoPE: whole frames from the start of the grid (their positions are those of the full grid)
    if cfg.sections is not None:
        t_len, h_len, w_len = cfg.grid
        frame = h_len * w_len
        frames, spent, elems = 1, 0.0, 0
        while True:
            tok = frames * frame
            qs, ks = f64(q_in[:, :tok]), f64(k_in[:, :tok])
            t0 = time.perf_counter()
            oracle.qk_norm_rope(qs, ks, f64(wq), f64(wk), (frames, h_len, w_len), cfg.sections, cfg.theta,
                                float(np.float32(cfg.eps)))
            spent = time.perf_counter() - t0
            elems = 2 * qs.size
            if spent > share["norm_rope"] * target_s / 4 or frames >= t_len:
                break
            frames = min(t_len, frames * 2)
        full = spent * (2 * b * n * hd * d) / elems
        stages["norm_rope"] = {"threads": 1, "seconds": spent, "sample": f"{frames} of {t_len} frames, all heads",
                               "gb_per_s": 8.0 * elems / 2 / spent / 1e9, "extrapolated_full_s": full}

    # selection: whole heads (pooling, scores, top-k), extrapolated over the heads
    spent, heads_done, sel = 0.0, 0, {}
    while heads_done < hd and (heads_done == 0 or spent < share["select"] * target_s):
        h = heads_done
        qs, ks = f64(q[:, :, h:h + 1]), f64(k[:, :, h:h + 1])
        t0 = time.perf_counter()
        sel[h] = oracle.subblock_select(qs, ks, 64, sparsity)
        spent += time.perf_counter() - t0
        heads_done += 1
    stages["select"] = {"threads": _blas_threads(), "seconds": spent, "sample": f"{heads_done} of {hd} heads, whole",
                        "extrapolated_full_s": spent * hd / heads_done}

    # dense and sparse attention: sampled query blocks of the heads selected above
    for name in ("dense", "sparse"):
        spent, rows_done, blocks, keys_done = 0.0, 0, 0, 0
        h = 0
        kh = vh = None
        while spent < share[name] * target_s and blocks < 64 * len(sel):
            if kh is None:
                kh, vh = f64(k[0, :, h]), f64(v[0, :, h])
            i = int(rng.integers(0, nb))
            rows = np.arange(i * 64, min(n, i * 64 + 64))
            qh = f64(q[0, rows, h])
            keys = slice(None) if name == "dense" else oracle.block_token_ids(sel[h][0, 0, i], 64, n)
            kk, vv = kh[keys], vh[keys]
            t0 = time.perf_counter()
            oracle.attention_head(qh, kk, vv)
            spent += time.perf_counter() - t0
            rows_done += len(rows)
            keys_done += len(rows) * kk.shape[0]
            blocks += 1
            if blocks % 16 == 0:
                h = (h + 1) % len(sel)
                kh = None
        flops = 4.0 * keys_done * d
        total = 4.0 * b * hd * n * n * d if name == "dense" else 4.0 * b * hd * nb * keep * 64 * 64 * d
        stages[name] = {"threads": _blas_threads(), "seconds": spent,
                        "sample": f"{blocks} query blocks ({rows_done} rows) of heads 0..{min(len(sel), hd) - 1}",
                        "tflops": flops / spent / 1e12, "extrapolated_full_s": spent * total / flops}

    step_flops = 4.0 * b * hd * n * n * d + 4.0 * b * hd * nb * keep * 64 * 64 * d
    step_s = sum(st["extrapolated_full_s"] for st in stages.values())
    measured = sum(st["seconds"] for st in stages.values())
    return {"value": step_flops / step_s / 1e12, "unit": "TFLOP/s",
            "cores": max(st["threads"] for st in stages.values()), "kind": "oracle",
            "sample": f"{cfg.name}: every oracle stage on a bounded sample ({measured:.1f} s measured), "
                      f"extrapolated to one whole step ({step_s:.0f} s extrapolated)",
            "seconds": measured, "extrapolated_step_s": step_s, "stages": stages,
            "cpu_model": _cpu_model(), "cpu_count": os.cpu_count(), "blas_threads": _blas_threads()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path (asked for {args.gpus}); "
              "the head-sharded layout it would use is described in the design notes.", file=sys.stderr)
        sys.exit(2)
    import video_diffusion_transformer_qk_amd as h3
    from inputs import CONFIGS, FRAME, TINY, VIDEO5S, VIDEO10S, VIDEO15S, make_inputs
    h3.load_library()
    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"generating workload {cfg.name} on {torch.cuda.get_device_name(dev)}")
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    x = make_inputs(cfg, dev)
    q, k, v, wq, wk = x["q"], x["k"], x["v"], x["wq"], x["wk"]
    b, n, hd, d = q.shape
    sections = cfg.sections
    nb = (n + 63) // 64
    keep = h3.keep_count(nb, args.sparsity)
    gs = args.group_stride if args.group_stride > 0 else h3.frame_group_stride(cfg.grid)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    out_d = torch.empty_like(q)
    out_s = torch.empty_like(q)
    idx = torch.empty((b, hd, nb, keep), dtype=torch.int32, device=dev)
    ws = torch.empty((h3.select_workspace_bytes(b, hd, n, d),), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # one pass of the hot path: norm+RoPE (pooling q', k' for the selection in the same pass),
    # dense attention, the selection on the pooled blocks, block-sparse attention
    pooled = {}

    def step(ev=None):
        if ev is not None: ev[0].record()
        pooled["p"] = h3.qk_norm_rope_pool(q, k, wq, wk, cfg.grid, sections, cfg.theta, cfg.eps, workspace=ws,
                                           out=(qo, ko))[2]
        if ev is not None: ev[1].record()
        h3.dense_fwd(qo, ko, v, out=out_d)
        if ev is not None: ev[2].record()
        h3.subblock_select_pooled(pooled["p"], args.sparsity, out=idx)
        if ev is not None: ev[3].record()
        h3.block_sparse_fwd(qo, ko, v, idx, out=out_s, group_stride=gs)
        if ev is not None: ev[4].record()

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    clocks = ClockSampler(enabled=not args.no_clock).start()
    start.record()
    for s in range(args.steps):
        step(events[s])
    end.record()
    torch.cuda.synchronize()
    clock = clocks.stop()
    wall = time.perf_counter() - t0
    ms_step = elapsed_ms(start, end) / args.steps
    per = {"norm_rope_pool": [], "dense": [], "select": [], "sparse": []}
    for ev in events:
        per["norm_rope_pool"].append(elapsed_ms(ev[0], ev[1]))
        per["dense"].append(elapsed_ms(ev[1], ev[2]))
        per["select"].append(elapsed_ms(ev[2], ev[3]))
        per["sparse"].append(elapsed_ms(ev[3], ev[4]))
    avg = {kname: float(np.mean(vals)) for kname, vals in per.items()}
    log(f"step {ms_step:.2f} ms (wall {wall / args.steps * 1e3:.2f} ms); per kernel " +
        ", ".join(f"{kk} {vv:.3f} ms" for kk, vv in avg.items()))

    dense_flops = 4.0 * b * hd * n * n * d
    sparse_flops = 4.0 * b * hd * nb * keep * 64 * 64 * d
    nr_bytes = 8.0 * b * n * hd * d
    # the pooled block statistics the fused pass also writes: per (tensor, batch, head, block) the
    # float64 means (8 D), their digits (3 D), exponent (4) and norms (8)
    pool_bytes = 2.0 * b * hd * nb * (11 * d + 12)
    dense_tf = dense_flops / (avg["dense"] * 1e-3) / 1e12
    sparse_tf = sparse_flops / (avg["sparse"] * 1e-3) / 1e12
    nrp_gbs = (nr_bytes + pool_bytes) / (avg["norm_rope_pool"] * 1e-3) / 1e9
    value = (dense_flops + sparse_flops) / (ms_step * 1e-3) / 1e12

    # the stand-alone calls on the same inputs: norm+RoPE alone, and the selection with its own
    # pooling pass (which also checks that the pooled path kept the same blocks)
    def median_ms(fn, reps=10, warm=2):
        ts = []
        for r in range(warm + reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if r >= warm:
                ts.append(elapsed_ms(e0, e1))
        return float(np.median(ts))
    idx_pooled = idx.clone()
    nr_ms = median_ms(lambda: h3.qk_norm_rope(q, k, wq, wk, cfg.grid, sections, cfg.theta, cfg.eps, out=(qo, ko)))
    sel_alone_ms = median_ms(lambda: h3.subblock_select(qo, ko, args.sparsity, workspace=ws, out=idx))
    same_sets = bool(torch.equal(idx, idx_pooled))
    nr_gbs = nr_bytes / (nr_ms * 1e-3) / 1e9
    # selection's algorithmic bytes: q' and k' read once (pooling), the kept indices written once. On
    # the pooled path its time is the pooled selection plus what pooling adds to the norm+RoPE pass
    sel_bytes = 4.0 * b * n * hd * d + 4.0 * b * hd * nb * keep
    sel_extra_ms = max(0.0, avg["norm_rope_pool"] - nr_ms)
    sel_total_ms = avg["select"] + sel_extra_ms
    sel_gbs = sel_bytes / (sel_total_ms * 1e-3) / 1e9
    log(f"norm+rope alone {nr_ms:.3f} ms ({nr_gbs:.0f} GB/s); norm+rope with pooling {avg['norm_rope_pool']:.3f} ms; "
        f"selection {avg['select']:.3f} ms after pooling ({sel_total_ms:.3f} ms with the pooling's share), "
        f"{sel_alone_ms:.3f} ms with its own pooling pass; same kept sets: {same_sets}")

    components = {
        "gfx_clock_during_steps": clock,
        # context only: the published peak assumes 2.4 GHz; the same MFMA rate at the clock read above
        "dense_frac_peak_at_measured_clock": (dense_tf / (PEAK_BF16_TFLOPS * clock["median_mhz"] / 2400.0)
                                              if clock else None),
        "step_kernel_ms": {kname: {"median": float(np.median(vals)), "min": float(np.min(vals)),
                                   "p90": float(np.percentile(vals, 90)), "mean": float(np.mean(vals))}
                           for kname, vals in per.items()},
        "dense_ms": avg["dense"], "dense_tflops": dense_tf, "dense_frac_peak": dense_tf / PEAK_BF16_TFLOPS,
        "sparse_ms": avg["sparse"], "sparse_tflops_kept": sparse_tf, "sparse_frac_peak": sparse_tf / PEAK_BF16_TFLOPS,
        # selection after the pooling in the norm+RoPE pass, and with the pooling's share of that pass
        "select_ms": avg["select"], "select_pool_share_ms": sel_extra_ms, "select_total_ms": sel_total_ms,
        "select_bytes": sel_bytes, "select_gbs": sel_gbs, "select_frac_peak": sel_gbs / PEAK_HBM_GBS,
        "select_standalone_ms": sel_alone_ms, "pooled_select_equals_standalone": same_sets,
        # norm+RoPE alone (same inputs, after the timed steps) and the step's pass that also pools
        "norm_rope_ms": nr_ms, "norm_rope_gbs": nr_gbs, "norm_rope_frac_peak": nr_gbs / PEAK_HBM_GBS,
        "norm_rope_pool_ms": avg["norm_rope_pool"], "norm_rope_pool_bytes": nr_bytes + pool_bytes,
        "norm_rope_pool_gbs": nrp_gbs, "norm_rope_pool_frac_peak": nrp_gbs / PEAK_HBM_GBS,
        "keep": keep, "n_blocks": nb,
        "dense_flops": dense_flops, "sparse_flops": sparse_flops, "norm_rope_bytes": nr_bytes,
    }

    if not args.no_extra:
        # norm+RoPE alone with MALL/L2 flushed before every run, at the 10 s and frame workloads
        flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
        for c2 in (VIDEO10S, FRAME):
            x2 = make_inputs(c2, dev)
            qq, kk2 = x2["q"], x2["k"]
            o1, o2 = torch.empty_like(qq), torch.empty_like(kk2)
            times = []
            for r in range(12):
                flush_caches(flush)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                h3.qk_norm_rope(qq, kk2, x2["wq"], x2["wk"], c2.grid, c2.sections, c2.theta, c2.eps, out=(o1, o2))
                e1.record()
                torch.cuda.synchronize()
                if r >= 2:
                    times.append(elapsed_ms(e0, e1))
            by = 8.0 * qq.numel()
            med = float(np.median(times))
            components[f"norm_rope_{c2.name}_us"] = med * 1e3
            components[f"norm_rope_{c2.name}_gbs"] = by / (med * 1e-3) / 1e9
            log(f"norm+rope {c2.name}: {med * 1e3:.1f} us median, {by / (med * 1e-3) / 1e9:.0f} GB/s (flushed)")
            if c2 is FRAME:
                # a single short launch between two events also times the events and the dispatch;
                # 60 back-to-back launches rotating over 6 input/output sets (6 x 99 MB, more than
                # the 256 MB MALL, so every launch reads from HBM) time the kernels themselves
                sets = [(qq.clone(), kk2.clone(), torch.empty_like(qq), torch.empty_like(kk2)) for _ in range(6)]
                per_launch = []
                for r in range(3):
                    flush_caches(flush)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for j in range(60):
                        a_, b_, c_, d_ = sets[j % 6]
                        h3.qk_norm_rope(a_, b_, x2["wq"], x2["wk"], c2.grid, c2.sections, c2.theta, c2.eps, out=(c_, d_))
                    e1.record()
                    torch.cuda.synchronize()
                    per_launch.append(elapsed_ms(e0, e1) / 60)
                bb = float(np.median(per_launch))
                components[f"norm_rope_{c2.name}_back_to_back_us"] = bb * 1e3
                components[f"norm_rope_{c2.name}_back_to_back_gbs"] = by / (bb * 1e-3) / 1e9
                log(f"norm+rope {c2.name}: {bb * 1e3:.1f} us per launch back to back over 6 sets, "
                    f"{by / (bb * 1e-3) / 1e9:.0f} GB/s ({by / (bb * 1e-3) / 1e9 / PEAK_HBM_GBS * 100:.1f} %)")
                del sets
            del x2, qq, kk2, o1, o2
        # the runtime's other fused block ops at this workload's shape: hidden = heads*head_dim
        # tokens wide, SwiGLU on a 4x-hidden MLP width (an assumed expansion ratio), flushed
        hidden = hd * d
        xa = torch.randn((b, n, hidden), device=dev, dtype=torch.float32).to(torch.bfloat16)
        sh = torch.randn((b, hidden), device=dev)
        scl = torch.randn((b, hidden), device=dev) * 0.1
        ya = torch.empty_like(xa)
        gate = torch.randn((b * n, 4 * hidden), device=dev, dtype=torch.bfloat16)
        up = torch.randn((b * n, 4 * hidden), device=dev, dtype=torch.bfloat16)
        ys = torch.empty_like(gate)
        rws = torch.empty((h3.load_library().h3attn_residual_workspace_bytes(xa.numel()),), dtype=torch.uint8, device=dev)
        rres = torch.empty((2,), dtype=torch.float64, device=dev)
        for name, fn, by in (("adaln", lambda: h3.adaln_modulate(xa, sh, scl, 1e-6, out=ya), 4.0 * xa.numel()),
                             ("swiglu", lambda: h3.swiglu(gate, up, out=ys), 6.0 * gate.numel()),
                             ("residual_change", lambda: h3.residual_change(xa, ya, workspace=rws, out=rres),
                              4.0 * xa.numel())):
            times = []
            for r in range(8):
                flush_caches(flush)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                if r >= 2:
                    times.append(elapsed_ms(e0, e1))
            med = float(np.median(times))
            components[f"{name}_us"] = med * 1e3
            components[f"{name}_gbs"] = by / (med * 1e-3) / 1e9
            components[f"{name}_frac_peak"] = by / (med * 1e-3) / 1e9 / PEAK_HBM_GBS
            log(f"{name}: {med * 1e3:.1f} us median, {by / (med * 1e-3) / 1e9:.0f} GB/s (flushed, {by / 1e9:.2f} GB)")
        del xa, ya, gate, up, ys, flush

    if not args.no_extra:
        # threshold mode (variable kept set per query block, CSR): tau bisected, outside any timed
        # region, so that about the same quarter of the key blocks is kept
        tws = torch.empty((h3.threshold_workspace_bytes(b, hd, n, d),), dtype=torch.uint8, device=dev)
        lo, hi = 0.0, 1.0
        while True:
            rp, _ = h3.subblock_select_threshold(qo, ko, hi, workspace=tws)
            if int(rp[-1].item()) >= 0.25 * rp.numel() * nb or hi > 1e6:
                break
            hi *= 2.0
        for _ in range(12):
            mid = 0.5 * (lo + hi)
            rp, _ = h3.subblock_select_threshold(qo, ko, mid, workspace=tws)
            if int(rp[-1].item()) > (1.0 - args.sparsity) * (rp.numel() - 1) * nb:
                hi = mid
            else:
                lo = mid
        tau = hi
        rp, ci = h3.subblock_select_threshold(qo, ko, tau, workspace=tws)
        out_c = torch.empty_like(q)
        h3.block_sparse_csr_fwd(qo, ko, v, rp, ci, out=out_c, group_stride=gs)
        torch.cuda.synchronize()
        nnz = int(rp[-1].item())
        tsel, tcsr = [], []
        for r in range(3):
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record()
            h3.subblock_select_threshold(qo, ko, tau, workspace=tws)   # includes one host read of nnz
            e1.record()
            h3.block_sparse_csr_fwd(qo, ko, v, rp, ci, out=out_c, group_stride=gs)
            e2.record()
            torch.cuda.synchronize()
            tsel.append(elapsed_ms(e0, e1))
            tcsr.append(elapsed_ms(e1, e2))
        csr_flops = 4.0 * nnz * 64 * 64 * d
        components["threshold_mode"] = {
            "tau": tau, "kept_fraction": nnz / ((rp.numel() - 1) * nb), "select_ms": float(np.median(tsel)),
            "csr_sparse_ms": float(np.median(tcsr)),
            "csr_sparse_tflops_kept": csr_flops / (float(np.median(tcsr)) * 1e-3) / 1e12}
        log(f"threshold mode: tau {tau:.4g}, kept {components['threshold_mode']['kept_fraction']:.3f}, select "
            f"{components['threshold_mode']['select_ms']:.2f} ms, csr sparse {components['threshold_mode']['csr_sparse_ms']:.2f} ms "
            f"({components['threshold_mode']['csr_sparse_tflops_kept']:.0f} TFLOP/s)")
        del tws, out_c

    if not args.no_extra:
        # fp8 (e4m3) path on the same inputs and kept sets: quantisation (an HBM stream; 3 bytes
        # per element of each of q, k, v: bf16 read, e4m3 written) and dense / block-sparse
        # attention on the quantised tensors, against the fp8 dense MFMA peak
        fws = torch.empty((h3.fp8_workspace_bytes(b, hd, n, d),), dtype=torch.uint8, device=dev)
        fq = h3.fp8_quantize(qo, ko, v, workspace=fws)
        out_f = torch.empty_like(q)
        h3.fp8_dense_fwd(fq, out=out_f)
        h3.fp8_block_sparse_fwd(fq, idx, out=out_f, group_stride=gs)
        torch.cuda.synchronize()
        tq, tdn, tsp = [], [], []
        for r in range(3):
            ev4 = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            ev4[0].record()
            h3.fp8_quantize(qo, ko, v, workspace=fws, out=fq)
            ev4[1].record()
            h3.fp8_dense_fwd(fq, out=out_f)
            ev4[2].record()
            h3.fp8_block_sparse_fwd(fq, idx, out=out_f, group_stride=gs)
            ev4[3].record()
            torch.cuda.synchronize()
            tq.append(elapsed_ms(ev4[0], ev4[1]))
            tdn.append(elapsed_ms(ev4[1], ev4[2]))
            tsp.append(elapsed_ms(ev4[2], ev4[3]))
        mq, md, msp = (float(np.median(t)) for t in (tq, tdn, tsp))
        qbytes = 9.0 * q.numel()
        components["fp8"] = {
            "quantize_ms": mq, "quantize_gbs": qbytes / (mq * 1e-3) / 1e9,
            "dense_ms": md, "dense_tflops": dense_flops / (md * 1e-3) / 1e12,
            "dense_frac_fp8_peak": dense_flops / (md * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
            "sparse_ms": msp, "sparse_tflops_kept": sparse_flops / (msp * 1e-3) / 1e12,
            "sparse_frac_fp8_peak": sparse_flops / (msp * 1e-3) / 1e12 / PEAK_FP8_TFLOPS}
        log(f"fp8: quantize {mq:.2f} ms ({components['fp8']['quantize_gbs']:.0f} GB/s), dense {md:.1f} ms "
            f"({components['fp8']['dense_tflops']:.0f} TFLOP/s), sparse {msp:.1f} ms "
            f"({components['fp8']['sparse_tflops_kept']:.0f} TFLOP/s kept)")
        del fws, fq, out_f

    if not args.no_extra:
        # the 10 s (12 heads, sparsity 0.75 and 0.80) and 15 s (12 heads, planted boxes, 0.75)
        # workloads: dense attention against selection + block-sparse attention, one warm-up and
        # the median of three runs each. The 10 s path starts with norm+RoPE; the 15 s path feeds
        # the synthetic q, k straight to attention and selection.
        del out_s, ws
        for c2 in (VIDEO10S, VIDEO15S):
            x2 = make_inputs(c2, dev)
            q2, k2, v2 = x2["q"], x2["k"], x2["v"]
            b2, n2, h2, d2 = q2.shape
            nb2 = (n2 + 63) // 64
            gs2 = h3.frame_group_stride(c2.grid)
            if c2 is VIDEO10S:
                q2n, k2n = torch.empty_like(q2), torch.empty_like(k2)
                h3.qk_norm_rope(q2, k2, x2["wq"], x2["wk"], c2.grid, c2.sections, c2.theta, c2.eps, out=(q2n, k2n))
                q2, k2 = q2n, k2n
            o2 = torch.empty_like(q2)
            ws2 = torch.empty((h3.select_workspace_bytes(b2, h2, n2, d2),), dtype=torch.uint8, device=dev)
            fl_dense = 4.0 * b2 * h2 * n2 * n2 * d2
            td = []
            for r in range(4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                h3.dense_fwd(q2, k2, v2, out=o2)
                e1.record()
                torch.cuda.synchronize()
                if r >= 1:
                    td.append(elapsed_ms(e0, e1))
            md = float(np.median(td))
            rec = {"n_tokens": n2, "heads": h2, "grid": list(c2.grid), "dense_ms": md,
                   "dense_tflops": fl_dense / (md * 1e-3) / 1e12, "group_stride": gs2}
            for sp in c2.sparsities:
                keep2 = h3.keep_count(nb2, sp)
                idx2 = torch.empty((b2, h2, nb2, keep2), dtype=torch.int32, device=dev)
                tsel, tsp = [], []
                for r in range(4):
                    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                    e0.record()
                    h3.subblock_select(q2, k2, sp, workspace=ws2, out=idx2)
                    e1.record()
                    h3.block_sparse_fwd(q2, k2, v2, idx2, out=o2, group_stride=gs2)
                    e2.record()
                    torch.cuda.synchronize()
                    if r >= 1:
                        tsel.append(elapsed_ms(e0, e1))
                        tsp.append(elapsed_ms(e1, e2))
                msel, msp = float(np.median(tsel)), float(np.median(tsp))
                fl_sp = 4.0 * b2 * h2 * nb2 * keep2 * 64 * 64 * d2
                rec[f"s{sp:.2f}"] = {"keep": keep2, "select_ms": msel, "sparse_ms": msp,
                                     "sparse_tflops_kept": fl_sp / (msp * 1e-3) / 1e12,
                                     "sparse_frac_peak": fl_sp / (msp * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                     "speedup_vs_dense": md / (msel + msp)}
                log(f"{c2.name}: dense {md:.1f} ms ({rec['dense_tflops']:.0f} TFLOP/s); sparsity {sp}: select "
                    f"{msel:.2f} ms + sparse {msp:.1f} ms ({rec[f's{sp:.2f}']['sparse_tflops_kept']:.0f} TFLOP/s "
                    f"kept), {md / (msel + msp):.2f}x faster than dense")
                del idx2
            components[c2.name] = rec
            del x2, q2, k2, v2, o2, ws2
        # the two small workloads (tiny 4x8x8 and one 48x84 frame): each call of the path timed 50
        # times (median, min, p90); launch-bound at these sizes, reported as context
        for c2 in (TINY, FRAME):
            x2 = make_inputs(c2, dev)
            q2, k2, v2 = x2["q"], x2["k"], x2["v"]
            b2, n2, h2, d2 = q2.shape
            sp = c2.sparsities[0]
            q2o, k2o, o2 = torch.empty_like(q2), torch.empty_like(k2), torch.empty_like(q2)
            ws2 = torch.empty((h3.select_workspace_bytes(b2, h2, n2, d2),), dtype=torch.uint8, device=dev)
            nb2 = (n2 + 63) // 64
            idx2 = torch.empty((b2, h2, nb2, h3.keep_count(nb2, sp)), dtype=torch.int32, device=dev)
            calls = {
                "norm_rope": lambda: h3.qk_norm_rope(q2, k2, x2["wq"], x2["wk"], c2.grid, c2.sections, c2.theta, c2.eps,
                                                     out=(q2o, k2o)),
                "dense": lambda: h3.dense_fwd(q2o, k2o, v2, out=o2),
                "select": lambda: h3.subblock_select(q2o, k2o, sp, workspace=ws2, out=idx2),
                "sparse": lambda: h3.block_sparse_fwd(q2o, k2o, v2, idx2, out=o2),
            }
            rec = {"sparsity": sp, "runs": 50}
            for nm, fn in calls.items():
                fn()
                torch.cuda.synchronize()
                ts = []
                for r in range(50):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    fn()
                    e1.record()
                    torch.cuda.synchronize()
                    ts.append(elapsed_ms(e0, e1) * 1e3)
                rec[f"{nm}_us"] = {"median": float(np.median(ts)), "min": float(np.min(ts)),
                                   "p90": float(np.percentile(ts, 90))}
            components[c2.name] = rec
            log(f"{c2.name}: " + ", ".join(f"{nm} {rec[nm + '_us']['median']:.1f} us" for nm in calls))
            del x2, q2, k2, v2, q2o, k2o, o2, ws2, idx2
        # context rates on the same device: a bf16 GEMM through torch (hipBLASLt) and a device copy
        a_m = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
        b_m = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
        c_m = torch.empty((8192, 8192), device=dev, dtype=torch.bfloat16)
        cp_src = torch.ones(1 << 30, dtype=torch.bfloat16, device=dev)   # 2 GiB
        cp_dst = torch.empty_like(cp_src)
        tg, tc = [], []
        for r in range(8):
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record()
            torch.matmul(a_m, b_m, out=c_m)
            e1.record()
            cp_dst.copy_(cp_src)
            e2.record()
            torch.cuda.synchronize()
            if r >= 2:
                tg.append(elapsed_ms(e0, e1))
                tc.append(elapsed_ms(e1, e2))
        gemm_tf = 2.0 * 8192 ** 3 / (float(np.median(tg)) * 1e-3) / 1e12
        copy_gbs = 2.0 * cp_src.numel() * 2 / (float(np.median(tc)) * 1e-3) / 1e9
        components["context"] = {"torch_matmul_bf16_8192_tflops": gemm_tf,
                                 "dense_frac_of_torch_matmul": dense_tf / gemm_tf,
                                 "device_copy_2gib_gbs": copy_gbs,
                                 "norm_rope_frac_of_copy": nr_gbs / copy_gbs}
        log(f"context: torch.matmul bf16 8192^3 {gemm_tf:.0f} TFLOP/s (dense attention at "
            f"{dense_tf / gemm_tf:.2f} of it); 2 GiB copy_ {copy_gbs:.0f} GB/s")
        del a_m, b_m, c_m, cp_src, cp_dst

    # the committed counters were taken on the 5 s workload; a run on another workload reports none
    dense_name = f"attn_fwd_kernel<{d},8,2> (dense)"
    traffic = measured_traffic(dense_name) if cfg is VIDEO5S else None
    roofline = {"bound": "mfma", "kernel": dense_name,
                "achieved": dense_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": dense_tf / PEAK_BF16_TFLOPS,
                "traffic": traffic,
                "traffic_unit": "bytes per launch (FETCH_SIZE x2.000 + WRITE_SIZE x1.000, copy-calibrated)",
                # one pass's figure above; the range over every recorded pass (the L2 hit rate varies)
                "traffic_observed_range": measured_traffic_range() if traffic is not None else None,
                "per_launch_flops": dense_flops, "avg_launch_ms": avg["dense"]}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on a bounded sample (host cores)")
        cpu = cpu_baseline(q, k, wq, wk, qo, ko, v, cfg, args.sparsity, args.cpu_seconds)
        log(f"cpu baseline {cpu['value']:.4g} TFLOP/s ({cpu['sample']}); stages "
            + ", ".join(f"{k_}: {st['seconds']:.1f} s -> {st['extrapolated_full_s']:.3g} s" for k_, st in cpu["stages"].items()))

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "batch": b, "heads": hd, "head_dim": d, "n_tokens": n,
                   "grid": list(cfg.grid), "sparsity": args.sparsity, "block_size": 64,
                   "group_stride": gs,
                   "step": "qk_norm_rope + dense_fwd + subblock_select + block_sparse_fwd"},
        "roofline": roofline, "cpu_baseline": cpu, "components": components,
        "provenance": provenance(cfg),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
