"""Comparison helpers for GPU-vs-oracle parity (no arithmetic of the method lives here)."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

# spec tolerances for bf16 attention outputs against the float64 oracle (N(0,1) inputs)
ATTN_MAX_ABS = 2e-2
ATTN_MEAN_ABS = 2e-3
# LSE (natural log). The kernels add up the bf16-rounded probabilities that P.V uses (each within
# 2^-9 relative), so ln(sum) may move by up to ln(1 + 2^-9) = 1.95e-3; the float32 logits (128
# exact products summed in float32) add up to D 2^-24 sum|q||k| / sqrt(D), about 1e-3 on the rows
# of the 15 s workload's planted high-norm keys. 4e-3 covers both.
LSE_MAX_ABS = 4e-3
NEAR_TIE_REL = 1e-5
# fp8 (e4m3) attention against exact float64 attention: q, k, v and the probabilities each carry
# 3 significant bits, so the bar is looser than the bf16 one. For the workloads' inputs
# (v ~ N(0,1)): absolute; measured worst 0.041 / 2.2e-3 on the frame workload and 0.125 / 3.2e-3
# on sampled 5 s blocks (the oracle's own fp8 rule against exact attention: 0.072 / 3.2e-3).
FP8_EXACT_MAX_ABS = 0.15
FP8_EXACT_MEAN_ABS = 1e-2
# For inputs whose token and channel magnitudes differ by powers of two (scores up to ~16), the
# error is taken relative to the RMS of each value channel over the keys; measured worst 0.74 /
# 0.016 on the ragged cases.
FP8_EXACT_MAX_REL_RMS = 1.5
FP8_EXACT_MEAN_REL_RMS = 3e-2


def log(msg: str):
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# One summary record per (workload, check), printed at the end of the pytest session by
# tests/conftest.py, so that the figures behind every pass are in the run's own output.
RECORDS = []


def record(workload: str, check: str, **fields):
    """Add or merge a summary record: numeric fields keep their worst value (max, except fields
    ending in _min which keep the min), counters (ints) add up."""
    for r in RECORDS:
        if r["workload"] == workload and r["check"] == check:
            for k, v in fields.items():
                if k not in r:
                    r[k] = v
                elif isinstance(v, bool) or isinstance(v, str):
                    r[k] = v
                elif isinstance(v, int):
                    r[k] += v
                elif k.endswith("_min"):
                    r[k] = min(r[k], v)
                else:
                    r[k] = max(r[k], v)
            return
    RECORDS.append({"workload": workload, "check": check, **fields})


def format_record(r) -> str:
    parts = []
    for k, v in r.items():
        if k in ("workload", "check"):
            continue
        parts.append(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}")
    return f"{r['workload']:>18s} {r['check']:<22s} " + " ".join(parts)


def host_bf16(t: torch.Tensor) -> torch.Tensor:
    """Device bf16 tensor -> host bf16 copy (the exact bytes the GPU consumed)."""
    return t.detach().to("cpu")


def f64(t: torch.Tensor) -> np.ndarray:
    """bf16/fp32 torch tensor (host or device) -> float64 numpy, exact."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits): 2^(floor(log2|x|) - 7)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def check_norm_rope(gpu: np.ndarray, ref: np.ndarray):
    """Each element within one bf16 ulp of the float64 value; near-zero results of a rotation
    (cancellation inside a pair) get an absolute floor of 2^-16 of the pair's magnitude.
    Returns (max error in ulps, fraction exactly equal to round-to-nearest of the reference)."""
    pair_mag = np.sqrt(ref[..., 0::2] ** 2 + ref[..., 1::2] ** 2)
    floor = np.repeat(pair_mag, 2, axis=-1) * 2.0 ** -16
    tol = np.maximum(bf16_ulp(ref), floor)
    err = np.abs(gpu - ref)
    worst = float(np.max(err / tol))
    rne = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    exact = float(np.mean(gpu == rne))
    return worst, exact


def check_attention(gpu: np.ndarray, ref: np.ndarray, what: str):
    d = np.abs(gpu - ref)
    mx, mean = float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    log(f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e}")
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    assert mx <= ATTN_MAX_ABS, f"{what}: max-abs {mx} > {ATTN_MAX_ABS}"
    assert mean <= ATTN_MEAN_ABS, f"{what}: mean-abs {mean} > {ATTN_MEAN_ABS}"
    return mx, mean


def check_block_sets(gpu_idx: np.ndarray, ref_idx: np.ndarray, scores: np.ndarray, keep: int, what: str):
    """Bit-exact per-row index sets, except rows whose keep-th and (keep+1)-th oracle scores are
    within NEAR_TIE_REL relative of each other; such mismatches are counted and reported."""
    import oracle
    nb = scores.shape[-1]
    assert gpu_idx.shape == ref_idx.shape, (gpu_idx.shape, ref_idx.shape)
    g = gpu_idx.reshape(-1, keep)
    r = ref_idx.reshape(-1, keep)
    # validity: ascending, unique, in range
    assert (g >= 0).all() and (g < nb).all(), f"{what}: index out of range"
    if keep > 1:
        assert (np.diff(g, axis=1) > 0).all(), f"{what}: rows not strictly ascending"
    mism = np.any(g != r, axis=1)
    near = oracle.near_tie_rows(scores, keep, NEAR_TIE_REL).reshape(-1)
    bad = mism & ~near
    log(f"{what}: rows {g.shape[0]}, mismatched {int(mism.sum())} (near-tie {int((mism & near).sum())}), "
        f"near-tie rows {int(near.sum())}")
    assert not bad.any(), f"{what}: {int(bad.sum())} non-near-tie rows differ, first row {int(np.argmax(bad))}"
    # in an excused row, only blocks whose scores tie with the keep-th score (within the same
    # relative band) may be swapped
    flat = scores.reshape(-1, nb)
    for row in np.nonzero(mism)[0]:
        kth = np.sort(flat[row])[::-1][keep - 1]
        for j in set(g[row].tolist()) ^ set(r[row].tolist()):
            assert abs(flat[row, j] - kth) <= NEAR_TIE_REL * max(abs(kth), abs(flat[row, j])), \
                f"{what}: row {row} swaps block {j} (score {flat[row, j]!r}) far from the keep-th score {kth!r}"
    return int(mism.sum()), int(near.sum())
