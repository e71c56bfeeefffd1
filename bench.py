#!/usr/bin/env python3
"""MLA prefill throughput on one MI355X (gfx950), through the C ABI of libmla_prefill.so.

One step = one full dense varlen MLA prefill call over the headline batch: the GPU tile planner,
the dense attention kernel and (when the split heuristic splits the keys) the combine kernel.
The headline batch is 8 sequences with lengths uniform in [64, 2048] (seeded), 128 heads, q/k
head 192 (128 nope + 64 rope), v head 128, bf16, causal, LSE on.

Printed: ONE JSON line with the throughput in TFLOP/s of algorithmic work (visible query-key
pairs x 640 FLOP x heads), the dense kernel's roofline position (its own device time from HIP
events recorded around each launch on its stream) and the fp64 CPU oracle timed on a bounded
sample of the same batch. "per_call" gives the median and minimum device time of single calls,
warm (back to back) and cold (a 1 GiB write evicts the caches before each call); "calibration"
gives this device's sustained rate of a pure bf16 MFMA loop and of a streaming HBM read, so the
kernels can be quoted against measured as well as published peaks. Secondary measurements of the other workloads (long context, chunked
prefill, sparse top-k, the 128-token case) are included under "secondary" unless
--no-secondary is given.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA prefill TFLOP/s (causal, varlen) + % bf16 MFMA peak on 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0     # MI355X published dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0         # MI355X published HBM3E bandwidth
DQK, DV = 192, 128
SP_D, SP_DV = 576, 512
PROFILES = os.path.join(ROOT, "profiles")
CALIB = {}                    # measured device rates (filled in by main unless --no-calib)


# ----------------------------------------------------------------------------- work counting
def dense_pairs(lens_q, lens_k, causal: bool, window=(-1, -1)) -> int:
    """Visible (query, key) pairs: bottom-right causal, an optional (left, right) window (-1 =
    unlimited, causal = right 0), or all pairs."""
    import numpy as np
    left, right = int(window[0]), int(window[1])
    if causal:
        right = 0
    total = 0
    for sq, sk in zip(lens_q, lens_k):
        i = np.arange(sq, dtype=np.int64)
        d = sk - sq
        hi = np.minimum(sk - 1, i + d + right) if right >= 0 else np.full(sq, sk - 1, dtype=np.int64)
        lo = np.maximum(0, i + d - left) if left >= 0 else np.zeros(sq, dtype=np.int64)
        total += int(np.maximum(hi - lo + 1, 0).sum())
    return total


def dense_flops(lens_q, lens_k, heads, causal, window=(-1, -1), dqk=DQK, dv=DV) -> float:
    return float(2 * (dqk + dv) * heads * dense_pairs(lens_q, lens_k, causal, window))


def dense_bytes(lens_q, lens_k, heads, lse=True, dqk=DQK, dv=DV, out_bytes=2) -> float:
    tq, tk = sum(lens_q), sum(lens_k)
    return float(tq * heads * dqk * 2 + tk * heads * (dqk + dv) * 2 + tq * heads * dv * out_bytes
                 + (tq * heads * 4 if lse else 0))


def sparse_flops(valid_slots, heads) -> float:
    return float(2 * (SP_D + SP_DV) * heads * valid_slots)


def sparse_bytes(valid_slots, tokens, heads, topk, lse=True) -> float:
    return float(valid_slots * SP_D * 2 + tokens * heads * SP_D * 2 + tokens * heads * SP_DV * 2
                 + tokens * topk * 4 + (tokens * heads * 4 if lse else 0))


def kernel_source_hash(kernel_file: str = "dense_fwd.hip") -> str:
    h = hashlib.sha256()
    for f in (kernel_file, "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "mla_varlen_prefill_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- timing helpers
def settle(step, ms: float = 100.0):
    """Run `step` back to back for about `ms` milliseconds. Right after an idle period the device
    runs at transient clocks for a few tens of milliseconds (step times first drop, then rise
    by up to 40 %, then settle), so secondary measurements start from the settled state."""
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            step()
        torch.cuda.synchronize()


def time_steps(step, steps: int, warmup: int, kernel: str):
    import torch
    import mla_varlen_prefill_amd as mla
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    mla.profile_enable(True, kinds=[kernel])  # events around the measured kernel only
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    k_ms, k_n = mla.profile_read(kernel)
    mla.profile_enable(False)
    return (t1 - t0) * 1e3 / steps, (k_ms / k_n if k_n else float("nan")), k_n


def per_call_ms(step, reps: int, flush=None):
    """Device milliseconds of single calls, each bracketed by events on the current stream. With
    `flush` (a large device buffer) every call is preceded by a write over it, which evicts the L2
    and the last-level cache, so the call starts cold."""
    import torch
    times = []
    for _ in range(reps):
        if flush is not None:
            flush.zero_()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        step()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    times.sort()
    return {"median_ms": round(times[len(times) // 2], 5), "min_ms": round(times[0], 5), "calls": reps}


def warm_cold(step, reps: int):
    import torch
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    res = {"warm": per_call_ms(step, reps), "cold_1GiB_flush": per_call_ms(step, reps, flush)}
    del flush
    torch.cuda.empty_cache()
    return res


def dense_device_case(name, lens_q, lens_k, heads, seed, steps, warmup, num_splits=0, window=None,
                      dqk=DQK, dv=DV, fp8_out=False, cpu_budget=0.0):
    """One dense workload timed through the C ABI; (dqk, dv) picks the head layout and fp8_out the
    FP8 output (static scale 2^-8). With cpu_budget > 0 the oracle is timed on a sample of the
    same inputs (cpu_rows_baseline) after the GPU measurements."""
    import torch
    import mla_varlen_prefill_amd as mla
    from workloads import device_dense
    q, k, v, cu_q, cu_k = device_dense(lens_q, lens_k, heads, seed, dqk=dqk, dv=dv)
    max_q, max_k = max(lens_q), max(lens_k)
    out = torch.empty((q.shape[0], heads, dv), dtype=torch.float8_e4m3fn if fp8_out else torch.bfloat16,
                      device="cuda")
    out_scale = torch.tensor([2.0 ** -8], dtype=torch.float32, device="cuda") if fp8_out else None
    lse = torch.empty((q.shape[0], heads), dtype=torch.float32, device="cuda")
    ws_bytes = mla.varlen_workspace_bytes(len(lens_q), q.shape[0], max_q, max_k, heads, True, num_splits, dv)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    scale = dqk ** -0.5

    def step():
        mla.mla_prefill_varlen(q, k, v, cu_q, cu_k, max_q, max_k, scale, causal=True,
                               num_splits=num_splits, out=out, lse=lse, workspace=ws, window=window,
                               out_scale=out_scale)

    settle(step)
    ms, kms, _ = time_steps(step, steps, warmup, "dense")
    wc = warm_cold(step, max(3, min(steps, 7)))
    fl = dense_flops(lens_q, lens_k, heads, True, window if window is not None else (-1, -1), dqk, dv)
    by = dense_bytes(lens_q, lens_k, heads, True, dqk, dv, 1 if fp8_out else 2)
    splits = mla.varlen_num_splits(len(lens_q), max_q, max_k, heads, True, num_splits, dqk, dv)
    cpu = None
    if cpu_budget > 0:
        cpu = cpu_rows_baseline(q, k, v, cu_q.cpu().numpy(), cu_k.cpu().numpy(), lens_q, lens_k, scale,
                                cpu_budget)
    del q, k, v, out, lse, ws, out_scale
    torch.cuda.empty_cache()
    res = {"workload": name, "ms_per_call": round(ms, 4), "dense_kernel_ms": round(kms, 4),
           "splits": splits, "tflops": round(fl / ms / 1e9, 2),
           "frac_bf16_peak": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
           "kernel_tflops": round(fl / kms / 1e9, 2), "alg_gbps": round(by / ms / 1e6, 1),
           "per_call": wc}
    if CALIB:
        res["frac_measured_mfma"] = round(fl / kms / 1e9 / CALIB["mfma_loop_tflops"], 4)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    return res


def dense_varlen_variant(name, steps, warmup, **kw):
    """The headline varlen batch (8 sequences, lengths in [64, 2048], 128 heads, causal) with
    another head layout or FP8 output."""
    from workloads import varlen_lens
    lens = varlen_lens(2, 8, 64, 2048)
    return dense_device_case(name, lens, lens, 128, 2, steps, warmup, **kw)


def sparse_case(steps, warmup, cpu_budget=0.0):
    import torch
    import mla_varlen_prefill_amd as mla
    from workloads import device_sparse
    t, h, n_kv, topk = 4096, 128, 65536, 2048
    q, kv, idx, sink, idx_host = device_sparse(t, h, n_kv, topk, seed=5)
    out = torch.empty((t, h, SP_DV), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((t, h), dtype=torch.float32, device="cuda")
    scale = SP_D ** -0.5

    def step():
        mla.mla_prefill_sparse(q, kv, idx, scale, sink=sink, out=out, lse=lse)

    settle(step)
    ms, kms, _ = time_steps(step, steps, warmup, "sparse")
    wc = warm_cold(step, max(3, min(steps, 7)))
    valid = int(((idx_host >= 0) & (idx_host < n_kv)).sum())
    fl = sparse_flops(valid, h)
    by = sparse_bytes(valid, t, h, topk)
    cpu = cpu_sparse_baseline(q, kv, idx_host, sink, scale, cpu_budget) if cpu_budget > 0 else None
    del q, kv, idx, out, lse
    torch.cuda.empty_cache()
    res = {"workload": "sparse_t4096_h128_topk2048_pool65536", "ms_per_call": round(ms, 4),
           "sparse_kernel_ms": round(kms, 4), "tflops": round(fl / ms / 1e9, 2),
           "frac_bf16_peak": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
           "alg_gbps": round(by / ms / 1e6, 1), "frac_hbm": round(by / ms / 1e6 / PEAK_HBM_GBS, 4),
           "kernel_alg_gbps": round(by / kms / 1e6, 1), "per_call": wc}
    res["traffic"] = measured_traffic("sparse_fwd_t4096_h128_topk2048_traffic.json", "sparse_fwd.hip")
    if CALIB:
        res["frac_measured_stream_read"] = round(by / kms / 1e6 / CALIB["stream_read_gbps"], 4)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    return res


def chunked_context_case(steps, warmup, chunk_tokens=4096):
    """The chunked-prefill shape with its context in a latent cache: 4 sequences of 2048 new tokens
    over 14336 / 10297 / 6143 / 2049 cached positions (so 16384 / 12345 / 8191 / 4097 keys in
    all), 128 heads; the context is up-projected chunk by chunk (W_KV ~ N(0, 1/512))."""
    import numpy as np
    import torch
    import mla_varlen_prefill_amd as mla
    from workloads import device_dense, device_randn_bf16, cu_from_lens
    new = [2048] * 4
    ctx = [n - 2048 for n in (16384, 12345, 8191, 4097)]
    h = 128
    q, k, v, cu_q, _ = device_dense(new, new, h, 4)
    latent = device_randn_bf16((sum(ctx), SP_D), 4, 9)
    w_kv = (device_randn_bf16((h * 256, 512), 4, 10).float() * 512 ** -0.5).to(torch.bfloat16)
    cu_c = torch.from_numpy(cu_from_lens(ctx)).cuda()
    out = torch.empty((q.shape[0], h, DV), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((q.shape[0], h), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(mla.chunked_context_workspace_bytes(4, q.shape[0], 2048, h, chunk_tokens), 16),
                     dtype=torch.uint8, device="cuda")

    def step():
        mla.mla_prefill_chunked_context(q, k, v, cu_q, latent, cu_c, w_kv, 2048, max(ctx), DQK ** -0.5,
                                        chunk_tokens=chunk_tokens, out=out, lse=lse, workspace=ws)

    settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    mla.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    kern = {name: mla.profile_read(name) for name in ("dense", "upproj", "combine")}
    mla.profile_enable(False)
    att = dense_flops(new, [c + n for c, n in zip(ctx, new)], h, True)
    up = 2.0 * sum(ctx) * h * 256 * 512
    del q, k, v, latent, w_kv, out, lse, ws
    torch.cuda.empty_cache()
    per_step = {name: round(t / steps, 4) for name, (t, n) in kern.items()}
    return {"workload": f"chunked_context_b4_q2048_ctx14336..2049_h128_chunk{chunk_tokens}",
            "ms_per_call": round(ms, 4), "attention_flop": att, "upproj_flop": up,
            "tflops_attention_plus_upproj": round((att + up) / ms / 1e9, 2),
            "kernel_ms_per_call": per_step,
            "upproj_tflops": round(up / (per_step["upproj"] * 1e9), 2) if per_step["upproj"] > 0 else None}


def sparse_paged_case(steps, warmup, block_size=64):
    """The sparse workload through a paged cache: the same latent rows scattered over shuffled
    pages of `block_size` rows, logical indices mapped through the block table in the kernel."""
    import torch
    import mla_varlen_prefill_amd as mla
    from workloads import device_sparse_paged
    t, h, n_kv, topk = 4096, 128, 65536, 2048
    q, kv, cache, table, cu_q, idx, sink, idx_host = device_sparse_paged(t, h, n_kv, topk, block_size, seed=5)
    del kv
    out = torch.empty((t, h, SP_DV), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((t, h), dtype=torch.float32, device="cuda")
    scale = SP_D ** -0.5

    def step():
        mla.mla_prefill_sparse_paged(q, cache, table, cu_q, idx, scale, sink=sink, out=out, lse=lse)

    settle(step)
    ms, kms, _ = time_steps(step, steps, warmup, "sparse")
    valid = int(((idx_host >= 0) & (idx_host < n_kv)).sum())
    by = sparse_bytes(valid, t, h, topk)
    del q, cache, idx, out, lse
    torch.cuda.empty_cache()
    return {"workload": f"sparse_paged_t4096_h128_topk2048_pool65536_bs{block_size}",
            "ms_per_call": round(ms, 4), "sparse_kernel_ms": round(kms, 4),
            "tflops": round(sparse_flops(valid, h) / ms / 1e9, 2),
            "alg_gbps": round(by / ms / 1e6, 1), "frac_hbm": round(by / ms / 1e6 / PEAK_HBM_GBS, 4)}


# ----------------------------------------------------------------------------- CPU baseline
def oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(q, k, v, lens, scale, budget_s: float):
    """The fp64 oracle, as it stands, on heads 0, 1, ... of the headline batch (all sequences,
    all rows) until the budget is spent. q/k/v are the device inputs; each head is copied to the
    host as bf16 bits before it is timed."""
    import numpy as np
    from oracle import mla_oracle as O
    from workloads import bf16_tensor_to_bits, cu_from_lens
    cu = cu_from_lens(lens)
    heads = q.shape[1]
    per_head = dense_flops(lens, lens, 1, True)
    done, el = 0, 0.0
    while done < heads and el < budget_s:
        qh, kh, vh = (bf16_tensor_to_bits(x[:, done:done + 1, :]) for x in (q, k, v))
        t0 = time.perf_counter()
        O.dense_mla_prefill(qh, kh, vh, cu, cu, scale, True)
        el += time.perf_counter() - t0
        done += 1
    return {"value": round(per_head * done / el / 1e12, 6), "unit": "TFLOP/s", "cores": oracle_threads(),
            "kind": "oracle",
            "sample": f"heads 0..{done - 1} of {heads} of the headline batch (all 8 sequences, all rows), "
                      f"{el:.1f} s of oracle time, fp64 numpy"}


def cpu_rows_baseline(q, k, v, cu_q, cu_k, lens_q, lens_k, scale, budget_s: float, head: int = 0):
    """The fp64 oracle's row evaluator on one head of a large dense workload: query rows spread
    evenly over every sequence, timed until the budget is spent. The rate counts the algorithmic
    work of the rows done (their visible keys x 640 FLOP); the full workload's oracle time is that
    work extrapolated at the measured rate."""
    import numpy as np
    from oracle import mla_oracle as O
    from workloads import bf16_tensor_to_bits
    cq, ck = np.asarray(cu_q), np.asarray(cu_k)
    qh, kh, vh = (bf16_tensor_to_bits(x[:, head:head + 1, :]) for x in (q, k, v))
    rng = np.random.default_rng(0)
    order = rng.permutation(int(cq[-1]))
    fl_done, el, n = 0.0, 0.0, 0
    for t in order:
        b = int(np.searchsorted(cq, t, side="right") - 1)
        sq, sk = int(cq[b + 1] - cq[b]), int(ck[b + 1] - ck[b])
        i = int(t) - int(cq[b])
        t0 = time.perf_counter()
        O.dense_mla_prefill_rows(qh, kh, vh, cq, ck, scale, True, [int(t)], [0])
        el += time.perf_counter() - t0
        fl_done += 2.0 * (qh.shape[2] + vh.shape[2]) * max(0, min(sk, i + sk - sq + 1))
        n += 1
        if el >= budget_s:
            break
    rate = fl_done / el
    total = dense_flops(lens_q, lens_k, q.shape[1], True)
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": oracle_threads(), "kind": "oracle",
            "extrapolated_full_s": round(total / rate, 1),
            "sample": f"{n} random query rows of head {head} (of {q.shape[1]}), {el:.1f} s of oracle time, "
                      f"fp64 numpy; full-workload time extrapolated at that rate"}


def cpu_sparse_baseline(q, kv, idx_host, sink, scale, budget_s: float):
    """The fp64 sparse oracle on random tokens of the sparse workload (all 128 heads each), until
    the budget is spent; rate in algorithmic TFLOP/s and GB/s of the sample."""
    import numpy as np
    from oracle import mla_oracle as O
    from workloads import bf16_tensor_to_bits
    kvh = bf16_tensor_to_bits(kv)
    sink_h = sink.cpu().numpy()
    n_kv = kvh.shape[0]
    t_all, heads = q.shape[0], q.shape[1]
    order = np.random.default_rng(0).permutation(t_all)
    el, n, valid = 0.0, 0, 0
    for t in order:
        qt = bf16_tensor_to_bits(q[int(t):int(t) + 1])
        it = idx_host[int(t):int(t) + 1]
        t0 = time.perf_counter()
        O.sparse_mla_prefill(qt, kvh, it, scale, dv=SP_DV, sink=sink_h)
        el += time.perf_counter() - t0
        valid += int(((it >= 0) & (it < n_kv)).sum())
        n += 1
        if el >= budget_s:
            break
    fl = sparse_flops(valid, heads)
    by = sparse_bytes(valid, n, heads, idx_host.shape[1])
    all_valid = int(((idx_host >= 0) & (idx_host < n_kv)).sum())
    return {"value": round(fl / el / 1e12, 6), "unit": "TFLOP/s", "alg_gbps": round(by / el / 1e9, 3),
            "cores": oracle_threads(), "kind": "oracle",
            "extrapolated_full_s": round(sparse_flops(all_valid, heads) / (fl / el), 1),
            "sample": f"{n} random tokens of {t_all} (all {heads} heads), {el:.1f} s of oracle time, fp64 numpy"}


# ----------------------------------------------------------------------------- traffic
def measured_traffic(summary: str = "dense_fwd_varlen_b8_h128_traffic.json",
                     kernel_file: str = "dense_fwd.hip"):
    """HBM bytes per kernel launch from a committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE scaled by a 1 GiB copy), if it was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash(kernel_file):
        return None
    return d.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first; about 40 are needed for the clocks to settle after idle")
    ap.add_argument("--no-secondary", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-calib", action="store_true",
                    help="skip measuring this device's MFMA-loop and streaming-read rates")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work on the headline batch")
    ap.add_argument("--cpu-budget-secondary", type=float, default=4.0,
                    help="seconds of oracle work on each of the 128-token, long-context, chunked-prefill "
                         "and sparse workloads")
    ap.add_argument("--only", default=None,
                    help="run one workload and print its line: dense_varlen, dense_long, dense_chunked, "
                         "dense_small, dense_window, dense_dims128, dense_dims256, dense_fp8, chunked_context, "
                         "sparse, sparse_paged, copy (a plain 1 GiB device copy for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path: run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import mla_varlen_prefill_amd as mla

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mla.load_library()

    if args.only == "copy":
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return

    if not args.no_calib and args.only in (None, "dense_varlen", "dense_long", "dense_chunked",
                                           "dense_small", "dense_window", "dense_dims128", "dense_dims256",
                                           "dense_fp8", "chunked_context", "sparse", "sparse_paged"):
        from mla_varlen_prefill_amd import calib
        CALIB["mfma_loop_tflops"] = round(calib.mfma_tflops(), 1)
        CALIB["stream_read_gbps"] = round(calib.stream_read_gbps(), 1)

    if args.only not in (None, "dense_varlen"):
        sec_runs = {
            "dense_long": lambda: dense_device_case("dense_long_1x32768_h128", [32768], [32768], 128, 3,
                                                    args.steps, args.warmup),
            "dense_chunked": lambda: dense_device_case("dense_chunked_b4_q2048", [2048] * 4,
                                                       [16384, 12345, 8191, 4097], 128, 4, args.steps,
                                                       args.warmup),
            "dense_small": lambda: dense_device_case("dense_small_1x128_h16", [128], [128], 16, 1,
                                                     args.steps, args.warmup),
            "sparse": lambda: sparse_case(args.steps, args.warmup),
            "sparse_paged": lambda: sparse_paged_case(args.steps, args.warmup),
            "chunked_context": lambda: chunked_context_case(args.steps, args.warmup),
            "dense_window": lambda: dense_device_case("dense_window_1x32768_h128_w4096", [32768], [32768], 128,
                                                      3, args.steps, args.warmup, window=(4096, -1)),
            "dense_dims128": lambda: dense_varlen_variant("dense_varlen_b8_h128_qk128_v128", args.steps,
                                                          args.warmup, dqk=128, dv=128),
            "dense_dims256": lambda: dense_varlen_variant("dense_varlen_b8_h128_qk256_v256", args.steps,
                                                          args.warmup, dqk=256, dv=256),
            "dense_fp8": lambda: dense_varlen_variant("dense_varlen_b8_h128_fp8_out", args.steps, args.warmup,
                                                      fp8_out=True),
        }
        print(json.dumps(sec_runs[args.only]()), flush=True)
        return

    # ---------------- headline: dense varlen batch of 8, lengths in [64, 2048], 128 heads. The
    # inputs are drawn on the device (no host-side generation just before the timing), and the
    # step is run back to back for ~100 ms before the warm-up steps, so that the timed steps
    # start from settled clocks whatever --warmup is.
    from workloads import device_dense, varlen_lens
    lens = varlen_lens(2, 8, 64, 2048)
    heads, batch = 128, len(lens)
    q, k, v, cu_q, cu_k = device_dense(lens, lens, heads, 2)
    max_q = max_k = max(lens)
    scale = float(np.float32(DQK ** -0.5))
    out = torch.empty((q.shape[0], heads, DV), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((q.shape[0], heads), dtype=torch.float32, device="cuda")
    ws_bytes = mla.varlen_workspace_bytes(batch, q.shape[0], max_q, max_k, heads, True, 0)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    splits = mla.varlen_num_splits(batch, max_q, max_k, heads, True, 0)

    def step():
        mla.mla_prefill_varlen(q, k, v, cu_q, cu_k, max_q, max_k, scale, causal=True,
                               num_splits=0, out=out, lse=lse, workspace=ws)

    settle(step)
    ms, dense_kernel_ms, launches = time_steps(step, args.steps, args.warmup, "dense")
    per_call = warm_cold(step, max(3, min(args.steps, 11)))
    flops = dense_flops(lens, lens, heads, True)
    value = flops / (ms / 1e3) / 1e12
    achieved = flops / (dense_kernel_ms / 1e3) / 1e12
    traffic = measured_traffic()
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense_varlen_b8_h128_causal_lse", "batch": batch, "seq_lens": lens,
                   "heads": heads, "head_dim_qk": DQK, "head_dim_v": DV, "causal": True, "lse": True,
                   "num_splits": splits, "algorithmic_flop_per_step": flops,
                   "frac_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "dense_fwd_kernel",
                     "kernel_ms": round(dense_kernel_ms, 5), "launches_timed": launches},
        "per_call": per_call,
        "calibration": dict(CALIB) or None,
    }
    if CALIB:
        result["roofline"]["frac_measured_mfma"] = round(achieved / CALIB["mfma_loop_tflops"], 4)
    result["cpu_baseline"] = None if args.no_cpu else cpu_baseline(q, k, v, lens, scale, args.cpu_budget)
    del q, k, v, out, lse, ws
    torch.cuda.empty_cache()

    if not args.no_secondary:
        sec = []
        ss, sw = max(2, min(args.steps, 5)), 2
        cb = 0.0 if args.no_cpu else args.cpu_budget_secondary
        sec.append(dense_device_case("dense_small_1x128_h16", [128], [128], 16, 1, args.steps, args.warmup,
                                     cpu_budget=cb))
        sec.append(dense_device_case("dense_long_1x32768_h128", [32768], [32768], 128, 3, ss, sw, cpu_budget=cb))
        sec.append(dense_device_case("dense_chunked_b4_q2048", [2048] * 4, [16384, 12345, 8191, 4097],
                                     128, 4, ss, sw, cpu_budget=cb))
        sec.append(dense_device_case("dense_window_1x32768_h128_w4096", [32768], [32768], 128, 3, ss, sw,
                                     window=(4096, -1)))
        for name, kw in (("dense_varlen_b8_h128_qk128_v128", dict(dqk=128, dv=128)),
                         ("dense_varlen_b8_h128_qk256_v256", dict(dqk=256, dv=256)),
                         ("dense_varlen_b8_h128_fp8_out", dict(fp8_out=True))):
            sec.append(dense_varlen_variant(name, max(5, min(args.steps, 50)), 10, **kw))
        sec.append(chunked_context_case(ss, sw))
        sec.append(sparse_case(ss, sw, cpu_budget=cb))
        sec.append(sparse_paged_case(ss, sw))
        result["secondary"] = sec

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
