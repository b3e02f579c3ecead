#!/usr/bin/env python3
"""KDA benchmark on one MI355X.

Headline: chunked-prefill tokens/s at T = 65,536 tokens, H = 32 heads, d_k = d_v = 128,
bfloat16 q/k/v/beta, fp32 log-decay, fp32 state and outputs, chunk 64 (one step = one full
prefill of that batch: decay factors, gated Gram matrices, UT transform, WY factors, the
sequential state pass and the epilogue).  In the same run: the batched decode step at
256 sequences x 32 heads (1000 consecutive in-place steps), reported as steps/s and HBM GB/s.

Timing: W untimed warmup steps, then exactly K steps bracketed by torch.cuda.synchronize();
per-kernel durations come from HIP events the library records around each of its kernel
launches on the call's stream (kda_timing_begin/kda_timing_end).  Inputs are resident in HBM
before timing starts.  Every timed run is parity-checked against the fp64 oracle on a sample.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix-core peak
# algorithmic bytes per unit (bf16 q/k/v/beta, fp32 g, fp32 o, fp32 state)
PREFILL_BYTES_PER_TOKEN_HEAD = 256 + 256 + 256 + 512 + 2 + 512          # 1794
PREP_BYTES_PER_TOKEN_HEAD = 256 + 256 + 512 + 2                         # q, k, g, beta read by the prep kernel
STATE_BYTES_PER_TOKEN_HEAD = 256 + 2 + 512                              # v, beta read, o written by the state pass
PREFILL_FLOP_PER_TOKEN_HEAD = 139264                                    # chunked form, d=128, C=64
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix-core peak
# chunked backward, per token-head: read q, k, v (bf16), g (fp32), beta (bf16), dL/do (fp32); write
# dq, dk, dv, dg (fp32) and dbeta (fp32)
BWD_BYTES_PER_TOKEN_HEAD = 3 * 256 + 512 + 2 + 512 + 4 * 512 + 4       # 3846


def bwd_flop_per_chunk(C, d):
    """Matrix products of one chunk's backward (d_k = d_v = d), 2 flop per multiply-add:
    16 C d^2  state-sized products: W S0, K'^T D (states entering each chunk); K' dS1, Q+^T dO,
              W^T dD (state gradients); D dS1^T, dO S0^T, dD S0^T (their gradients)
    14 C^2 d  in-chunk products (triangular ones at half size): P, M, W, U; M^T dO; dM; dT (two);
              T^T dD, T^T dW; the four pairwise contractions of dP and dM
    C^3       the inverse T and dA = -T^T dT T^T"""
    return 16 * C * d * d + 14 * C * C * d + C ** 3
DECODE_BYTES_PER_SEQ_HEAD = 65536 + 65536 + 768 + 512 + 2 + 512         # 132866


# HBM traffic per launch measured with rocprofv3 --pmc (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch), scaled by the factors a plain device copy of known size reads for the same counters.
# Each entry holds the SHA-256 of the kernel source it was measured on; once that source changes
# the figure no longer describes the kernel and is reported as null.
# Figures and commands: profiles/hbm_counter_calibration_copy_1GiB.md, profiles/*_T65536_*.md,
# profiles/decode_N256_*.md.
COUNTER_SCALE = {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
_KIB = 1024
_MFMA_SRC = "gated_delta_rule_75_amd/csrc/kda_chunk_mfma.hip"
_MFMA_SHA = "6c4a05405bdcb1d57d471965b4de7627f2eb4e3f956caac226f03ae2219e73cb"
_DECODE_SRC = "gated_delta_rule_75_amd/csrc/kda_decode.hip"
_DECODE_SHA = "8f6da261804d588a7c98da378838a326741fe49876b995ac0c4a84bf7b3318b3"
_BWD_SRC = "gated_delta_rule_75_amd/csrc/kda_chunk_bwd.hip"
_BWD_SHA = "f1543487f96d6ce26799a14ce5f61491ee8107969deb57afc14457435247bf76"


def _counted(fetch_kib, write_kib):
    return round(fetch_kib * _KIB * COUNTER_SCALE["FETCH_SIZE"] + write_kib * _KIB * COUNTER_SCALE["WRITE_SIZE"])


# kernel name -> where and on what it was measured, and HBM bytes per launch
MEASURED_TRAFFIC = {
    "kda_prep": {"source": _MFMA_SRC, "sha256": _MFMA_SHA, "workload": "prefill T=65536 H=32",
                 "bytes": _counted(1065120.0, 1983493.2)},
    "kda_state": {"source": _MFMA_SRC, "sha256": _MFMA_SHA, "workload": "prefill T=65536 H=32",
                  "bytes": _counted(1271087.6, 1050785.0)},
    "kda_decode": {"source": _DECODE_SRC, "sha256": _DECODE_SHA, "workload": "decode N=256 H=32",
                   "bytes": _counted(267359.5, 528576.9)},
    # the five backward kernels of one pass (factors, fwd_chain, rev_chain, grad_state, grad_chunk)
    "kda_backward": {"source": _BWD_SRC, "sha256": _BWD_SHA, "workload": "backward T=65536 H=32",
                     "bytes": _counted(3422889.8 + 1601701.1 + 2378565.3 + 3704807.7 + 8924465.5,
                                       8270730.2 + 3372507.2 + 3161753.2 + 3687807.8 + 4414699.4)},
}


def source_sha256(rel):
    import hashlib

    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_of(kernel, workload=None):
    """Counter-derived HBM bytes per launch of `kernel`, or None if not measured on this source
    and workload."""
    m = MEASURED_TRAFFIC.get(kernel)
    if not m or (workload is not None and m["workload"] != workload) or source_sha256(m["source"]) != m["sha256"]:
        return None
    return m["bytes"]


# prefill MFMA utilisation from rocprofv3 --pmc MfmaUtil (percent of cycles the matrix cores are
# busy, per kernel), on the kernel source named by its SHA-256 (profiles/prefill_mfma_utilisation_*)
MEASURED_MFMA_UTIL = {"source": _MFMA_SRC, "sha256": _MFMA_SHA, "workload": "prefill T=65536 H=32",
                      "kda_prep": 0.081, "kda_state": 0.101}
# the algorithmic MFMA fraction at the HBM roofline: 139,264 flop per 1,794 B at 8 TB/s = 621
# TFLOP/s, 24.8% of the dense fp16/bf16 peak
MFMA_CEILING_AT_HBM_ROOFLINE = PREFILL_FLOP_PER_TOKEN_HEAD / PREFILL_BYTES_PER_TOKEN_HEAD * HBM_PEAK_GBPS / 1e3 / \
    MFMA_F16_PEAK_TFLOPS


def copy_rate(n=1 << 30, reps=5):
    """GB/s of a plain device-to-device copy of n bytes (n read + n written), best of reps, timed
    with events: the practical streaming ceiling of this machine's HBM."""
    import torch

    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best = None
    # torch's copy_ and its elementwise kernel (neg, vectorised loads and stores): the faster
    for fn in (lambda: dst.copy_(src), lambda: torch.neg(src, out=dst)):
        for _ in range(2):
            fn()
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n / (best * 1e-3) / 1e9


class CacheFlush:
    """Evicts the L2 caches and the 256 MB Infinity Cache by writing a 1 GiB buffer (untimed)."""

    def __init__(self):
        import torch

        self.buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        self.i = 0

    def __call__(self):
        self.i += 1
        self.buf.fill_(self.i & 0xFF)


def copy_calibration():
    """A plain device-to-device copy of 1 GiB: reads and writes exactly 2^30 bytes per launch."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dst.copy_(src)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    log(f"[copy] {n} B read + {n} B written in {dt * 1e3:.3f} ms ({2 * n / dt / 1e9:.1f} GB/s)")
    print(json.dumps({"copy_bytes": n, "ms": dt * 1e3, "GBps": 2 * n / dt / 1e9}), flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed prefill steps")
    ap.add_argument("--warmup", type=int, default=20, help="untimed prefill passes first (the clocks settle within about 20)")
    ap.add_argument("--T", type=int, default=65536, help="prefill tokens")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--decode-warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--skip-backward", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=3, help="timed chunked-backward passes")
    ap.add_argument("--skip-workloads", action="store_true",
                    help="skip the varlen append and long-context workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (the HBM-counter calibration kernel) and exit")
    return ap.parse_args()


def upload(x, dtype, device):
    import numpy as np
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def slice_err(x, y):
    """max over heads of max|x-y| / max|y| over the head's slice; x, y [T, H, dv]."""
    import numpy as np

    d = np.abs(x - y).max(axis=(0, 2))
    m = np.abs(y).max(axis=(0, 2))
    return float((d / np.where(m > 0, m, 1)).max())


def pass_traffic(workload):
    """HBM bytes of one prefill pass (both kernels) from the counters, or None."""
    parts = [traffic_of("kda_prep", workload), traffic_of("kda_state", workload)]
    return None if any(p is None for p in parts) else sum(parts)


def bench_prefill(args, res):
    import numpy as np
    import torch

    import gated_delta_rule_75_amd as kda
    import synth

    dev = torch.device("cuda:0")
    w = synth.workload("metric")
    T, H, dk, dv = args.T, w.H, w.dk, w.dv
    log(f"[prefill] generating T={T} H={H} d={dk} bf16 inputs")
    q, k, v, g, b = synth.gen_tokens(w, T)
    tq, tk, tv, tb = (upload(x, "bf16", dev).reshape(1, T, *x.shape[1:]) for x in (q, k, v, b))
    tg = upload(g, "f32", dev).reshape(1, T, H, dk)
    out = torch.empty((1, T, H, dv), dtype=torch.float32, device=dev)
    sT = torch.empty((1, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_size(0, 1, T, H, dk, dv, torch.bfloat16, 64), dtype=torch.uint8, device=dev)

    def step():
        kda.prefill_chunked(tq, tk, tv, tg, tb, None, out=out, state_out=sT, workspace=ws)

    log(f"[prefill] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[prefill] timing {args.steps} steps")
    # one pass = one kda_prefill_chunked call; its kernels may run on two streams, and the call's
    # stream (torch's current stream) waits for all of them, so events on it bracket the pass
    # The timed passes carry only these events; the per-kernel times come from the same number of
    # passes right after, with events around each launch (between the pass's two kernels they would
    # add stream commands to the timed passes).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    pass_list = [e0.elapsed_time(e1) for e0, e1 in evs]
    with kda.kernel_timing() as kt:
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
    per = {}
    for name, ms in kt.records:
        per.setdefault(name, []).append(ms)
    avg = {n: sum(x) / len(x) for n, x in per.items()}
    th = T * H
    path_ms = sum(pass_list) / len(pass_list)
    achieved = PREFILL_BYTES_PER_TOKEN_HEAD * th / (path_ms * 1e-3) / 1e9
    kernels = []
    for name, alg in (("kda_prep", PREP_BYTES_PER_TOKEN_HEAD), ("kda_state", STATE_BYTES_PER_TOKEN_HEAD)):
        if name in avg:
            launches = len(per[name]) // args.steps
            kernels.append({"kernel": name, "launches_per_pass": launches, "avg_ms_per_launch": round(avg[name], 4),
                            "ms_per_pass": round(avg[name] * launches, 4),
                            "algorithmic_bytes_per_pass": alg * th,
                            "traffic_per_pass": traffic_of(name, f"prefill T={T} H={H}"),
                            "achieved_GBps": round(alg * th / (avg[name] * launches * 1e-3) / 1e9, 1)})
    tflops = PREFILL_FLOP_PER_TOKEN_HEAD * th / (path_ms * 1e-3) / 1e12
    mfma_util = None
    if source_sha256(MEASURED_MFMA_UTIL["source"]) == MEASURED_MFMA_UTIL["sha256"] and \
            MEASURED_MFMA_UTIL["workload"] == f"prefill T={T} H={H}":
        mfma_util = {k: MEASURED_MFMA_UTIL[k] for k in ("kda_prep", "kda_state")}
    # cache-flush check: the same passes with L2 and the Infinity Cache evicted before each one
    flush = CacheFlush()
    fl = []
    for _ in range(min(args.steps, 10)):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        fl.append(e0.elapsed_time(e1))
    del flush
    torch.cuda.empty_cache()
    flushed_ms = sum(fl) / len(fl)
    res["value"] = T * args.steps / elapsed
    res["ms_per_step"] = elapsed * 1e3 / args.steps
    res["roofline"] = {
        "bound": "hbm", "kernel": "one prefill pass: kda_prep and kda_state over all segments",
        "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": pass_traffic(f"prefill T={T} H={H}"),
        "algorithmic_bytes_per_launch": PREFILL_BYTES_PER_TOKEN_HEAD * th,
        "avg_pass_ms": round(path_ms, 4), "min_pass_ms": round(min(pass_list), 4),
        "timing": "HIP events on the call's stream around each kda_prefill_chunked call (a pass) of the timed loop; the per-kernel times come from as many passes right after it, with events around each launch",
        "cache_flush": {"unflushed_avg_pass_ms": round(path_ms, 4), "flushed_avg_pass_ms": round(flushed_ms, 4),
                        "flushed_passes": len(fl),
                        "how": "1 GiB buffer written (untimed) before each flushed pass; the timed steps above run "
                               "back to back without it (each pass moves 8 GB, 32x the 256 MB Infinity Cache)"},
        "mfma_algorithmic_tflops": round(tflops, 1),
        "mfma_frac_of_f16_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
        "mfma_util_counters": mfma_util,
        "mfma_target_frac": 0.5, "mfma_target_met": False,
        "mfma_algorithmic_ceiling_at_hbm_roofline": round(MFMA_CEILING_AT_HBM_ROOFLINE, 4),
        "mfma_note": "the chunked prefill does 139,264 flop per 1,794 B (77.6 flop/B, below the fp16 ridge of "
                     "~313), so even at the full 8 TB/s its algorithmic matrix-core fraction is capped at the "
                     "ceiling above; the HBM-roofline fraction is the governing figure",
    }
    res["kernels"] = kernels
    kp = ", ".join(f"{x['kernel']}: {x['ms_per_pass']}" for x in kernels)
    log(f"[prefill] {res['value'] / 1e6:.2f} M tokens/s, {res['ms_per_step']:.3f} ms/step, pass {path_ms:.3f} ms "
        f"(events), kernel time per pass {{{kp}}}; with a cache flush before each pass {flushed_ms:.3f} ms")

    # the next rows on the same inputs: one gate per head (Gated DeltaNet: the first channel's
    # log-decay of each token) and state snapshots every 16 chunks
    tgh = tg[..., 0].contiguous()
    snaps = torch.empty((1, T // (16 * 64), H, dk, dv), dtype=torch.float32, device=dev)

    def timed_passes(fn):
        for _ in range(args.warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in ev) / len(ev)

    ms_head = timed_passes(lambda: kda.prefill_chunked(tq, tk, tv, tgh, tb, None, out=out, state_out=sT,
                                                       workspace=ws))
    ms_snap = timed_passes(lambda: kda.prefill_chunked(tq, tk, tv, tg, tb, None, out=out, state_out=sT,
                                                       workspace=ws, snapshot_every=16, snapshots=snaps))
    head_bytes = (PREFILL_BYTES_PER_TOKEN_HEAD - 512 + 4) * th  # g is one fp32 per token-head
    res["next_rows"] = {
        "head_gate_prefill": {"workload": f"as the headline, g [T,H] (one log-decay per token and head)",
                              "ms_per_pass": round(ms_head, 4), "tokens_per_s": round(T / (ms_head * 1e-3), 1),
                              "roofline": {"bound": "hbm", "achieved": round(head_bytes / (ms_head * 1e-3) / 1e9, 1),
                                           "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                           "frac": round(head_bytes / (ms_head * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                           "algorithmic_bytes_per_launch": head_bytes}},
        "snapshots_every_16_chunks": {"snapshots": int(snaps.shape[1]), "ms_per_pass": round(ms_snap, 4),
                                      "overhead_vs_headline": round(ms_snap / path_ms - 1, 4)},
    }
    log(f"[prefill] per-head gate {ms_head:.3f} ms/pass; with {snaps.shape[1]} snapshots {ms_snap:.3f} ms/pass")
    del snaps, tgh

    # parity of the timed output on a token sample (all heads) + CPU baseline from the same oracle run
    step()
    torch.cuda.synchronize()
    wide_all = (q, k, v, g, b)
    return out, sT, wide_all


def oracle_sample(args, res, out, wide_all):
    import numpy as np

    import oracle
    import synth

    q, k, v, g, b = wide_all
    H = q.shape[1]
    threads = oracle.default_threads()

    def run(Ts):
        sl = slice(0, Ts)
        ins = [synth.to_f64(q[sl], "bf16"), synth.to_f64(k[sl], "bf16"), synth.to_f64(v[sl], "bf16"),
               g[sl].astype(np.float64), synth.to_f64(b[sl], "bf16")]
        t0 = time.perf_counter()
        o, s = oracle.recurrence(*ins, threads=threads)
        return o, time.perf_counter() - t0

    _, tc = run(256)
    rate = 256 / max(tc, 1e-6)
    Ts = int(min(q.shape[0], max(512, rate * args.cpu_seconds)))
    Ts = max(64, Ts - Ts % 64)
    log(f"[oracle] calibration {rate:.0f} tokens/s on {threads} threads; sample {Ts} tokens x {H} heads")
    o_ref, t = run(Ts)
    o_gpu = out[0, :Ts].detach().cpu().numpy().astype(np.float64)
    err = slice_err(o_gpu, o_ref)
    # one host thread, on a smaller sample of the same tokens
    T1 = 256
    ins1 = [synth.to_f64(q[:T1], "bf16"), synth.to_f64(k[:T1], "bf16"), synth.to_f64(v[:T1], "bf16"),
            g[:T1].astype(np.float64), synth.to_f64(b[:T1], "bf16")]
    t0 = time.perf_counter()
    oracle.recurrence(*ins1, threads=1)
    t1 = time.perf_counter() - t0
    res["cpu_baseline"] = {"value": round(Ts / t, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                           "sample": f"first {Ts} tokens x {H} heads of the T={q.shape[0]} prefill workload "
                                     f"(fp64 token recurrence, {t:.1f} s)",
                           "threads": threads, "host_cores": host_cores(), "os_cpu_count": os.cpu_count(),
                           "threads_note": "the oracle runs on at most 16 threads, the host CPU share of one GPU "
                                           "on this machine; host_cores is what the process may run on",
                           "single_core": {"value": round(T1 / t1, 2), "unit": "tokens/s", "threads": 1,
                                           "sample": f"first {T1} tokens x {H} heads, {t1:.2f} s"}}
    res["parity"] = {"prefill_tokens_checked": Ts, "heads": H, "max_slice_rel_err": err, "tol": 2e-3,
                     "ok": bool(err <= 2e-3)}
    log(f"[oracle] {Ts / t:.1f} tokens/s; parity max err {err:.2e}")


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def oracle_rates(args, res):
    """The oracle's rate on the other workloads' own inputs (bounded samples, every head), on the
    same host threads and on one thread: the prefill workload (T=8192), the varlen append workload
    (the first tokens of each of its 8 segments, from their carried states) and the long-context
    workload (its first tokens; and its decode tail, one token per step on all heads)."""
    import numpy as np

    import oracle
    import synth

    threads = oracle.default_threads()

    def timed(ins, cu=None, s0=None, th=threads):
        t0 = time.perf_counter()
        o, sT = oracle.recurrence(*ins, cu, s0, threads=th)
        return time.perf_counter() - t0, sT

    def widen(x):
        q, k, v, g, b = x
        return [synth.to_f64(q, "bf16"), synth.to_f64(k, "bf16"), synth.to_f64(v, "bf16"), g.astype(np.float64),
                synth.to_f64(b, "bf16")]

    out = {}
    for name, n_all, n_one in (("prefill", 2048, 256), ("long", 2048, 256)):
        w = synth.workload(name)
        ins = widen(synth.gen_tokens(w, n_all))
        t_all, sT = timed(ins)
        t_one, _ = timed([x[:n_one] for x in ins], th=1)
        out[name] = {"tokens_per_s": round(n_all / t_all, 1), "threads": threads,
                     "single_core_tokens_per_s": round(n_one / t_one, 1),
                     "sample": f"first {n_all} tokens x {w.H} heads ({n_one} on one thread) of T={w.T}"}
        if name == "long":
            steps = 256
            dins = widen(synth.gen_tokens(w, steps, offset_tokens=n_all))
            # one sequence, one token per decode step, in order from the sample's final state
            t_dec, _ = timed(dins, None, sT, th=1)
            out["long_decode_tail"] = {"steps_per_s": round(steps / t_dec, 1), "threads": 1,
                                       "sample": f"{steps} decode steps (B=1, {w.H} heads) from the state after "
                                                 f"the first {n_all} tokens"}
    w = synth.workload("varlen")
    s0 = synth.gen_state(w, len(w.lengths))
    rates = []
    for n_seg, th in ((512, threads), (32, 1)):
        parts = [synth.gen_tokens(w, min(L, n_seg), offset_tokens=int(o))
                 for L, o in zip(w.lengths, synth.cu_seqlens(w.lengths)[:-1])]
        ins = widen([np.concatenate([p[i] for p in parts]) for i in range(5)])
        cu = synth.cu_seqlens([min(L, n_seg) for L in w.lengths])
        t, _ = timed(ins, cu, s0, th=th)
        rates.append(round(int(cu[-1]) / t, 1))
    out["varlen"] = {"tokens_per_s": rates[0], "threads": threads, "single_core_tokens_per_s": rates[1],
                     "sample": f"first 512 tokens (32 on one thread) of each of the {len(w.lengths)} segments x "
                               f"{w.H} heads, from their carried states"}
    res.setdefault("cpu_baseline", {})["per_workload"] = out
    log(f"[oracle] per workload: {out}")


def bench_backward(args, res, wide_all):
    """The chunked backward (training) on the headline prefill's inputs: one pass = one
    kda_chunked_backward call over all T tokens and H heads with dL/do ~ N(0, 1), dL/dS_T = 0 and
    a zero initial state.  Parity: one head's gradients on the last tokens, against the oracle's
    derivative started from the oracle's own state at that point."""
    import numpy as np
    import torch

    import gated_delta_rule_75_amd as kda
    import oracle
    import synth

    dev = torch.device("cuda:0")
    w = synth.workload("metric")
    q, k, v, g, b = wide_all
    T, H, d = q.shape[0], w.H, w.dk
    C = 64
    d_out, _ = synth.gen_cotangents(w, T, 1)
    tq, tk, tv, tb = (upload(x, "bf16", dev) for x in (q, k, v, b))
    tg, tdo = upload(g, "f32", dev), upload(d_out, "f32", dev)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    ws = torch.empty(kda.workspace_size(3, 1, T, H, d, d, torch.bfloat16, C), dtype=torch.uint8, device=dev)

    def step():
        return kda.chunked_backward(tq, tk, tv, tg, tb, cu, None, d_out=tdo, chunk=C, state_grad=False,
                                    workspace=ws)

    log(f"[backward] T={T} H={H} d={d}: warmup 1, timing {args.backward_steps} passes "
        f"(workspace {ws.numel() / 2**30:.1f} GiB)")
    step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.backward_steps)]
    with kda.kernel_timing() as kt:
        for e0, e1 in ev:
            e0.record()
            grads = step()
            e1.record()
        torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    avg_ms = sum(ms) / len(ms)
    per = {}
    for name, t in kt.records:
        per.setdefault(name, []).append(t)
    kernels = {n: round(sum(x) / args.backward_steps, 4) for n, x in per.items()}
    th = T * H
    flop = bwd_flop_per_chunk(C, d) * (T // C) * H
    nbytes = BWD_BYTES_PER_TOKEN_HEAD * th
    tflops = flop / (avg_ms * 1e-3) / 1e12
    gbps = nbytes / (avg_ms * 1e-3) / 1e9
    # parity: head 0, last n tokens; the oracle's state entering them from its own forward run
    n, h = 1024, 0
    wide = [synth.to_f64(q[:, h:h + 1], "bf16"), synth.to_f64(k[:, h:h + 1], "bf16"),
            synth.to_f64(v[:, h:h + 1], "bf16"), g[:, h:h + 1].astype(np.float64),
            synth.to_f64(b[:, h:h + 1], "bf16")]
    t0 = time.perf_counter()
    _, s_mid = oracle.recurrence(*(x[:T - n] for x in wide), threads=1)
    ref = oracle.backward(*(x[T - n:] for x in wide), None, s_mid, d_o=d_out[T - n:, h:h + 1], threads=1)
    t_or = time.perf_counter() - t0
    err = 0.0
    for x, y in zip(grads[:5], ref[:5]):
        xg = x[T - n:, h:h + 1].detach().cpu().numpy().astype(np.float64)
        err = max(err, float(np.abs(xg - y).max() / max(np.abs(y).max(), 1e-30)))
    res["next_rows"]["chunked_backward"] = {
        "workload": f"gradients of the headline prefill (T={T}, H={H}, d={d}, chunk {C}, bf16 inputs, fp32 "
                    "arithmetic); dL/do ~ N(0,1)",
        "arithmetic": "fp32 accumulation; at d=128, chunk 64 with bf16 inputs the chain and state-side products "
                      "take split-bf16 operands (hi + lo, three bf16 matrix-core steps per product, about 2^-18 "
                      "relative), the rest fp32 matrix-core steps",
        "ms_per_pass": round(avg_ms, 3), "min_pass_ms": round(min(ms), 3),
        "tokens_per_s": round(T / (avg_ms * 1e-3), 1), "kernels_ms_per_pass": kernels,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F32_PEAK_TFLOPS, 4),
                     "algorithmic_flop_per_launch": flop, "dtype": "f32"},
        "hbm": {"achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes_per_launch": nbytes,
                "traffic": traffic_of("kda_backward", f"backward T={T} H={H}")},
        "parity": {"head": h, "last_tokens": n, "max_rel_err": err, "tol": 2e-3, "ok": bool(err <= 2e-3),
                   "oracle_s": round(t_or, 1)},
    }
    log(f"[backward] {avg_ms:.3f} ms/pass ({T / (avg_ms * 1e-3) / 1e6:.2f} M tokens/s), {tflops:.1f} TFLOP/s "
        f"fp32 algorithmic, kernels {kernels}; parity {err:.2e}")


def bench_decode(args, res):
    import numpy as np
    import torch

    import gated_delta_rule_75_amd as kda
    import oracle
    import synth
    from gated_delta_rule_75_amd import _lib

    dev = torch.device("cuda:0")
    w = synth.workload("decode")
    N, H, dk, dv, steps = w.decode_N, w.H, w.dk, w.dv, args.decode_steps
    total = args.decode_warmup + steps
    log(f"[decode] generating N={N} H={H} d={dk}, {total} steps of inputs + state")
    q, k, v, g, b = synth.gen_tokens(w, total * N)
    s0 = synth.gen_state(w, N)
    tq, tk, tv, tb = (upload(x, "bf16", dev).reshape(total, N, *x.shape[1:]) for x in (q, k, v, b))
    tg = upload(g, "f32", dev).reshape(total, N, H, dk)
    S = upload(s0, "f32", dev)
    out = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    L = _lib.load()
    stream = torch.cuda.current_stream(dev).cuda_stream
    args_list = [(tq[i].data_ptr(), tk[i].data_ptr(), tv[i].data_ptr(), tg[i].data_ptr(), tb[i].data_ptr())
                 for i in range(total)]
    sp, op = S.data_ptr(), out.data_ptr()

    def step(i):
        rc = L.kda_decode_step(*args_list[i], sp, sp, op, N, H, dk, dv, _lib.KDA_BF16, stream)
        if rc:
            _lib.check(rc)

    for i in range(args.decode_warmup):
        step(i)
    torch.cuda.synchronize()
    # the wall-clock loop runs without per-launch timing events (they add two stream commands per
    # step); the kernel times come from a second pass over the same steps' inputs on a copy of the
    # state, so the timed run's in-place state, which the parity check below follows, is untouched
    Sk = S.clone()
    log(f"[decode] timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.decode_warmup, total):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    outk = torch.empty_like(out)
    skp, okp = Sk.data_ptr(), outk.data_ptr()
    with kda.kernel_timing() as kt:
        for i in range(args.decode_warmup, total):
            rc = L.kda_decode_step(*args_list[i], skp, skp, okp, N, H, dk, dv, _lib.KDA_BF16, stream)
            if rc:
                _lib.check(rc)
        torch.cuda.synchronize()
    del Sk, outk
    ms = [m for n, m in kt.records if n == "kda_decode"]
    avg = sum(ms) / len(ms)
    bytes_step = DECODE_BYTES_PER_SEQ_HEAD * N * H
    gbps_wall = steps * bytes_step / elapsed / 1e9
    gbps_kernel = bytes_step / (avg * 1e-3) / 1e9
    # cache-flush check: steps with L2 and the Infinity Cache evicted before each one (the 512 MiB
    # state is only twice the Infinity Cache, so the unflushed loop could read part of it from
    # there).  Out of place into a second state and output buffer (the same bytes moved), so that
    # the timed run's in-place state and last output, which the parity check below follows, are
    # left as they are.
    flush = CacheFlush()
    S2, out2 = torch.empty_like(S), torch.empty_like(out)
    sp2, op2 = S2.data_ptr(), out2.data_ptr()
    fl = []
    for i in range(args.decode_warmup, min(total, args.decode_warmup + 50)):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = L.kda_decode_step(*args_list[i], sp, sp2, op2, N, H, dk, dv, _lib.KDA_BF16, stream)
        e1.record()
        if rc:
            _lib.check(rc)
        torch.cuda.synchronize()
        fl.append(e0.elapsed_time(e1))
    del flush, S2, out2
    torch.cuda.empty_cache()
    flushed = sum(fl) / len(fl)
    res["decode"] = {"workload": f"decode step, {N} sequences x {H} heads, d={dk}, in-place fp32 state",
                     "steps": steps, "steps_per_s": round(steps / elapsed, 1),
                     "ms_per_step": round(elapsed * 1e3 / steps, 4), "hbm_GBps": round(gbps_wall, 1),
                     "kernel_avg_ms": round(avg, 4),
                     "cache_flush": {"flushed_step_ms": round(flushed, 4), "flushed_steps": len(fl),
                                     "flushed_GBps": round(bytes_step / (flushed * 1e-3) / 1e9, 1),
                                     "how": "1 GiB buffer written (untimed) before each flushed step (out of place, "
                                            "the same bytes), timed with events around the step; the 1000 timed "
                                            "steps run back to back in place"},
                     "timing": "steps_per_s: wall clock around the 1000 in-place steps with no per-launch events; "
                               "kernel_avg_ms: HIP events around each launch in a second pass over the same inputs "
                               "on a copy of the state"}
    res["roofline_decode"] = {"bound": "hbm", "kernel": "kda_decode", "achieved": round(gbps_kernel, 1),
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps_kernel / HBM_PEAK_GBPS, 4),
                              "traffic": traffic_of("kda_decode", f"decode N={N} H={H}"), "algorithmic_bytes_per_launch": bytes_step}
    log(f"[decode] {steps / elapsed:.1f} steps/s, {gbps_wall:.1f} GB/s wall, kernel avg {avg * 1e3:.1f} us "
        f"({gbps_kernel:.1f} GB/s); flushed step {flushed * 1e3:.1f} us")

    if args.no_cpu_baseline:
        return
    # CPU-baseline leg: the oracle steps sampled (sequence, head) pairs through every step
    # (warmup included); its results also check the timed run
    pairs = [(0, 0), (17, 5), (128, 31), (255, 12)]
    t_or = 0.0
    Sg = S.detach().cpu().numpy()
    og = out.detach().cpu().numpy()
    worst = 0.0
    for n, h in pairs:
        sl = lambda x: x.reshape(total, N, H, -1)[:, n, h, :]  # noqa: E731
        qi = synth.to_f64(sl(q), "bf16")[:, None, :]
        ki = synth.to_f64(sl(k), "bf16")[:, None, :]
        vi = synth.to_f64(sl(v), "bf16")[:, None, :]
        gi = sl(g).astype(np.float64)[:, None, :]
        bi = synth.to_f64(b.reshape(total, N, H)[:, n, h], "bf16")[:, None]
        t0 = time.perf_counter()
        o_ref, s_ref = oracle.recurrence(qi, ki, vi, gi, bi, None, s0[n, h][None, None].astype(np.float64))
        t_or += time.perf_counter() - t0
        es = np.abs(Sg[n, h] - s_ref[0, 0]).max() / np.abs(s_ref[0, 0]).max()
        eo = np.abs(og[n, h] - o_ref[-1, 0]).max() / np.abs(o_ref[-1, 0]).max()
        worst = max(worst, es, eo)
    res["parity"] = dict(res.get("parity", {}), decode_pairs_checked=len(pairs), decode_steps_checked=total,
                         decode_max_rel_err=float(worst), decode_ok=bool(worst <= 2e-3))
    # one (sequence, head) step is 1/(N*H) of a batch step
    res.setdefault("cpu_baseline", {})["decode"] = {
        "value": round(len(pairs) * total / t_or / (N * H), 3), "unit": "steps/s (batch 256 x 32 heads)",
        "sample": f"{len(pairs)} (sequence, head) pairs x {total} steps, single-threaded fp64 recurrence",
        "cores": 1}
    log(f"[decode] parity max err {worst:.2e}")


def _events_ms(fn, n):
    """Average ms of n calls of fn, each bracketed by HIP events on the current stream."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in ev) / n


def _head_err(x, y):
    import numpy as np

    return float(np.abs(x - y).max() / max(np.abs(y).max(), 1e-300))


def bench_workloads(args, res):
    """The varlen append workload (8 carried segments of 1K-32K tokens) and the long-context one
    (a 2^20-token prefill, then 4096 decode steps of the same sequence), each parity-checked on one
    sampled head against the oracle."""
    import numpy as np
    import torch

    import gated_delta_rule_75_amd as kda
    import oracle
    import synth

    dev = torch.device("cuda:0")
    out = {}
    # ---- varlen append-prefill from carried states
    w = synth.workload("varlen")
    cu = synth.cu_seqlens(w.lengths)
    T, N, H, dk, dv = int(cu[-1]), len(w.lengths), w.H, w.dk, w.dv
    log(f"[varlen] generating T_total={T} in {N} segments, H={H}")
    q, k, v, g, b = synth.gen_tokens(w, T)
    s0 = synth.gen_state(w, N)
    tq, tk, tv, tb = (upload(x, "bf16", dev) for x in (q, k, v, b))
    tg, ts0 = upload(g, "f32", dev), upload(s0, "f32", dev)
    tcu = torch.from_numpy(cu).to(dev)
    o = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
    sT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_size(1, N, T, H, dk, dv, torch.bfloat16, 64), dtype=torch.uint8, device=dev)

    def step():
        kda.append_prefill(tq, tk, tv, tg, tb, tcu, ts0, out=o, state_out=sT, workspace=ws)

    step()
    torch.cuda.synchronize()
    ms = _events_ms(step, 5)
    nbytes = PREFILL_BYTES_PER_TOKEN_HEAD * T * H + 2 * N * H * dk * dv * 4
    h = 5
    wide = [synth.to_f64(x[:, h:h + 1], "bf16") for x in (q, k, v)] + [g[:, h:h + 1].astype(np.float64),
                                                                       synth.to_f64(b[:, h:h + 1], "bf16")]
    t0 = time.perf_counter()
    oref, sref = oracle.recurrence(*wide, cu, s0[:, h:h + 1], vcols=32)
    t_or = time.perf_counter() - t0
    err = max(_head_err(o[:, h:h + 1].cpu().numpy().astype(np.float64), oref),
              _head_err(sT[:, h:h + 1].cpu().numpy().astype(np.float64), sref))
    out["varlen_append"] = {
        "workload": f"append-prefill of {N} segments ({T} tokens, lengths {list(map(int, w.lengths))}) "
                    f"from carried fp32 states, H={H}, d=128, bf16, chunk 64",
        "ms_per_pass": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "algorithmic_bytes_per_launch": nbytes},
        "parity": {"head": h, "all_tokens_and_states": True, "max_rel_err": err, "tol": 2e-3,
                   "ok": bool(err <= 2e-3), "oracle_s": round(t_or, 1)}}
    log(f"[varlen] {ms:.3f} ms/pass ({T / (ms * 1e-3) / 1e6:.2f} M tokens/s); parity {err:.2e}")
    del tq, tk, tv, tb, tg, ts0, o, sT, ws, q, k, v, g, b, wide, oref
    torch.cuda.empty_cache()

    # ---- long context: 2^20-token prefill, then decode steps from its final state
    w = synth.workload("long")
    T, H, steps = w.T, w.H, w.decode_steps
    log(f"[long] generating T={T} H={H}")
    q, k, v, g, b = synth.gen_tokens(w, T)
    tq, tk, tv, tb = (upload(x, "bf16", dev).reshape(1, T, *x.shape[1:]) for x in (q, k, v, b))
    tg = upload(g, "f32", dev).reshape(1, T, H, dk)
    o = torch.empty((1, T, H, dv), dtype=torch.float32, device=dev)
    sT = torch.empty((1, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_size(0, 1, T, H, dk, dv, torch.bfloat16, 64), dtype=torch.uint8, device=dev)

    def lstep():
        kda.prefill_chunked(tq, tk, tv, tg, tb, None, out=o, state_out=sT, workspace=ws)

    lstep()
    torch.cuda.synchronize()
    ms = _events_ms(lstep, 2)
    nbytes = PREFILL_BYTES_PER_TOKEN_HEAD * T * H
    del tq, tk, tv, tb, tg, ws
    torch.cuda.empty_cache()
    dq, dk_, dv_, dg, db = synth.gen_tokens(w, steps, offset_tokens=T)
    sq, sk, sv, sb = (upload(x, "bf16", dev) for x in (dq, dk_, dv_, db))
    sg = upload(dg, "f32", dev)
    S = sT.clone()
    dout = torch.empty((1, H, dv), dtype=torch.float32, device=dev)
    # each step's token tensors as views made before the timed loop (a caller has them at hand)
    toks = [(sq[t:t + 1], sk[t:t + 1], sv[t:t + 1], sg[t:t + 1], sb[t:t + 1]) for t in range(steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(steps):
        kda.decode_step(*toks[t], S, out=dout)
    e1.record()
    torch.cuda.synchronize()
    dms = e0.elapsed_time(e1)
    # per-kernel times from the library's event timing (two events around every launch, which slow
    # the host loop), on a copy of the state so that the timed steps above stay the checked ones
    Sk, kout = sT.clone(), torch.empty_like(dout)
    with kda.kernel_timing() as kt:
        for t in range(min(steps, 512)):
            kda.decode_step(sq[t:t + 1], sk[t:t + 1], sv[t:t + 1], sg[t:t + 1], sb[t:t + 1], Sk, out=kout)
        torch.cuda.synchronize()
    kus = [m * 1e3 for n, m in kt.records if n == "kda_decode"]
    del Sk, kout, toks
    # the first G of those steps captured in a HIP graph and replayed: time per step on the GPU with
    # no host call between the kernels; one replay is first checked bitwise against the same steps run
    # eagerly
    G = 64
    Sg, Se = sT.clone(), sT.clone()
    gout, eout = torch.empty_like(dout), torch.empty_like(dout)

    def gsteps(state, o_):
        for t in range(G):
            kda.decode_step(sq[t:t + 1], sk[t:t + 1], sv[t:t + 1], sg[t:t + 1], sb[t:t + 1], state, out=o_)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gsteps(Sg, gout)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gsteps(Sg, gout)
    Sg.copy_(sT)
    graph.replay()
    gsteps(Se, eout)
    torch.cuda.synchronize()
    graph_same = bool(torch.equal(Sg, Se) and torch.equal(gout, eout))
    reps = 20
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    gus = e0.elapsed_time(e1) * 1e3 / (reps * G)
    del graph, Sg, Se
    h = 11
    log(f"[long] oracle on head {h}")
    wide = [synth.to_f64(x[:, h:h + 1], "bf16") for x in (q, k, v)] + [g[:, h:h + 1].astype(np.float64),
                                                                       synth.to_f64(b[:, h:h + 1], "bf16")]
    t0 = time.perf_counter()
    oref, sref = oracle.recurrence(*wide, vcols=8)
    dwide = [synth.to_f64(x[:, h:h + 1], "bf16") for x in (dq, dk_, dv_)] + [
        dg[:, h:h + 1].astype(np.float64), synth.to_f64(db[:, h:h + 1], "bf16")]
    doref, dsref = oracle.recurrence(*dwide, None, sref, vcols=8)
    t_or = time.perf_counter() - t0
    err = max(_head_err(o[0, :, h:h + 1].cpu().numpy().astype(np.float64), oref),
              _head_err(sT[:, h:h + 1].cpu().numpy().astype(np.float64), sref),
              _head_err(dout[:, h:h + 1].cpu().numpy().astype(np.float64), doref[-1:]),
              _head_err(S[:, h:h + 1].cpu().numpy().astype(np.float64), dsref))
    out["long_context"] = {
        "workload": f"B=1 prefill of T={T} tokens, H={H}, d=128, bf16, chunk 64, then {steps} decode steps "
                    f"(B=1) from its final state",
        "prefill_ms_per_pass": round(ms, 3), "prefill_tokens_per_s": round(T / (ms * 1e-3), 1),
        "prefill_roofline": {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
                             "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                             "algorithmic_bytes_per_launch": nbytes},
        "decode_steps": steps, "decode_us_per_step": round(dms * 1e3 / steps, 2),
        "decode_steps_per_s": round(steps / (dms * 1e-3), 1),
        "decode_kernel_avg_us": round(sum(kus) / len(kus), 2),
        "decode_graph_us_per_step": round(gus, 2),
        "decode_graph_matches_eager": graph_same,
        "decode_note": "one sequence: each head's state split over 8 workgroups of 16 columns (256 per "
                       "step); bound by launch and memory latency, not by HBM.  decode_us_per_step includes "
                       "the host's calls through the Python binding (no timing events in that loop); "
                       "decode_kernel_avg_us is timed with HIP events around each launch over a separate "
                       "loop of up to 512 steps (the events add their own overhead); "
                       "decode_graph_us_per_step is the time per step of 64 steps replayed back to back "
                       "from a HIP graph",
        "parity": {"head": h, "prefill_tokens_checked": T, "decode_steps_checked": steps, "max_rel_err": err,
                   "tol": 2e-3, "ok": bool(err <= 2e-3), "oracle_s": round(t_or, 1)}}
    log(f"[long] prefill {ms:.2f} ms ({T / (ms * 1e-3) / 1e6:.2f} M tokens/s), decode {dms * 1e3 / steps:.1f} "
        f"us/step (kernel {sum(kus) / len(kus):.1f} us with events, {gus:.2f} us per step from a graph, "
        f"graph == eager: {graph_same}); parity {err:.2e}")
    res["workloads"] = out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU (it has no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    res = {
        "metric": "KDA prefill tokens/s (d=128, T=64K) + decode steps/s & HBM GB/s at batch 256",
        "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16-mfma/f32", "storage_dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; shapes and distributions of the workloads)",
        "config": {"workload": f"KDA chunked prefill B=1 T={args.T} H=32 d_k=d_v=128 chunk=64, bf16 q/k/v/beta, "
                               "fp32 log-decay/state/output; plus decode 256 seq x 32 heads x 1000 steps",
                   "global_batch": 1, "seq_len": args.T, "heads": 32, "head_dim": 128, "chunk": 64},
    }
    res["copy_GBps"] = round(copy_rate(), 1)
    res["copy_note"] = "best of 5 plain 1 GiB device-to-device streams (1 GiB read + 1 GiB written; torch copy_ " \
                       "and torch.neg), events: this box's practical HBM streaming rate; the roofline peak stays " \
                       "the 8 TB/s spec"
    log(f"[copy] {res['copy_GBps']} GB/s")
    out = None
    if not args.skip_prefill:
        out, sT, wide_all = bench_prefill(args, res)
        if not args.no_cpu_baseline:
            oracle_sample(args, res, out, wide_all)
            oracle_rates(args, res)
        del out, sT
        torch.cuda.empty_cache()
        if not args.skip_backward:
            bench_backward(args, res, wide_all)
        del wide_all
        torch.cuda.empty_cache()
    if not args.skip_decode:
        bench_decode(args, res)
    if not args.skip_workloads:
        torch.cuda.empty_cache()
        bench_workloads(args, res)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
