"""Benchmark: accumulated-rotation causal attention forward on one MI355X.

One step = the whole hot path on one batch of the 16x-extrapolation workload
(B=2, H=8, L=16384, d=64, bf16, learned token-dependent angles, rotation of
q, k and v): angle scan -> rotation pass -> attention kernel, through the C
ABI, with inputs resident in HBM.  Prints ONE JSON line.

  value         whole-step throughput in TFLOP/s of algorithmic attention
                work, 4 d per causal (query, key) pair (the two contractions)
  tokens_per_s  B * L / step time
  roofline      the attention kernel (the dominant one) against the bf16
                matrix-core peak; its duration is measured with HIP events on
                the stream it is launched on.  traffic = HBM bytes per launch
                from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary in
                profiles/, when that summary was taken on the current kernel
                source (else null)
  scan_roofline the angle scan against the HBM peak (8 bytes per element)
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
                workload (strided query rows of every head)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk/CU (dense)
HBM_PEAK_GBS = 8000.0
METRIC = "accum-rotation causal attention fwd TFLOP/s + tokens/s at L=16K, d=64"
CSRC = os.path.join(ROOT, "accumulated_rotation_positional_amd", "csrc")
ATTN_SOURCES = ("attn_bf16.hip", "arp_device.hpp", "mfma_tile.hpp")
SCAN_SOURCES = ("angle_scan.hip",)
COUNTERS = os.path.join(ROOT, "profiles", "attn_fwd_extrap_16k_hbm_counters.json")
FWD_COUNTERS = os.path.join(ROOT, "profiles", "forward_counters.json")
F32_SOURCES = ("attn_f32.hip", "arp_device.hpp")
# One wave64 vector instruction occupies a SIMD for 4 cycles (16 lanes): 256 CUs x
# 4 SIMDs x 2.4 GHz / 4 = 6.144e11 wave instructions per second.
VALU_PEAK_INSTS = 256 * 4 * 2.4e9 / 4


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--clock-warmup-s", type=float, default=1.0,
                   help="fixed untimed phase of whole steps run before the --warmup steps, "
                        "so that the timed steps see the clocks the GPU holds under this load")
    p.add_argument("--workload", default="extrap_16k")
    p.add_argument("--fused", action="store_true", help="rotate k/v inside the attention kernel")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-workloads", action="store_true",
                   help="skip the forward figures of the other workloads (profiling runs use "
                        "this so that each kernel's counters come from the headline workload)")
    p.add_argument("--forward-only", action="store_true",
                   help="only the timed forward steps of --workload (profiling runs of one "
                        "workload's forward kernels)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target duration of the CPU oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one plain device copy of 256 MiB (the reference kernel "
                        "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return p.parse_args()


def source_hash(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the attention kernel and of the angle scan from
    the committed counter summary; each is None when the summary is missing,
    was taken on another workload, or is older than that kernel's source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None, None
    if c.get("workload") != workload:
        return None, None
    attn = c.get("hbm_bytes_per_launch") if c.get("source_hash") == source_hash(ATTN_SOURCES) else None
    scan = (c.get("scan_hbm_bytes_per_launch")
            if c.get("scan_source_hash") == source_hash(SCAN_SOURCES) else None)
    return attn, scan


def forward_counters(key: str):
    """An entry of the committed per-workload counter summary, or None when it is
    missing or older than the sources of the kernel it describes."""
    try:
        with open(FWD_COUNTERS) as f:
            c = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if c is None:
        return None
    if "attn_source_hash" in c:
        src = ATTN_SOURCES if "attn_bf16" in c["attn_kernel"] else F32_SOURCES
        if c["attn_source_hash"] != source_hash(src):
            return None
    if "source_hash" in c and c["source_hash"] != source_hash(SCAN_SOURCES):
        return None
    return c


def _strided_rows(w, stride: int, offset: int = 0) -> np.ndarray:
    L = w.seqlen
    i = np.arange(offset % stride, L, stride, dtype=np.int64)
    return np.concatenate([bh * L + i for bh in range(w.batch * w.heads)])


def _parity_rows(w, total: int = 1024) -> np.ndarray:
    """About `total` query rows of a workload spread over all its heads: per
    head, evenly spaced rows plus the head's last (longest) row."""
    L, bh = w.seqlen, w.batch * w.heads
    per = max(1, total // bh)
    i = np.unique(np.concatenate([(np.arange(per, dtype=np.int64) * L) // per + (7 % max(L // per, 1)),
                                  [L - 1]]))
    i = i[i < L]
    return np.concatenate([h * L + i for h in range(bh)])


def run_workload_parity(samples: dict) -> dict:
    """Each other workload's timed output against the oracle on sampled rows
    (the oracle recomputes each head's angle scan and rotation at full
    length): max |error| beside the bar and the relative rms error."""
    import oracle
    from accumulated_rotation_positional_amd import workloads as wl
    out = {}
    for name, (rows, got) in samples.items():
        w = wl.make(name)
        flags = (oracle.ROTATE_QK | (oracle.ROTATE_V if w.rotate_v else 0) |
                 (oracle.ALIBI if w.use_alibi else 0))
        t0 = time.perf_counter()
        ref = oracle.Problem(w.q, w.k, w.v, w.phi, flags, alibi=w.alibi).rows(rows, host_threads())
        out[name] = {**_parity(got, ref, 2e-2 if w.dtype == "bf16" else 1e-4),
                     "oracle_seconds": round(time.perf_counter() - t0, 2)}
    return out


def run_cpu_baseline(w, flags: int, alibi, target_s: float, got=None) -> dict:
    """Time the oracle on strided query rows.  Its cost is a fixed part per
    head (angle scan and key/value rotation) plus a part per row, so two
    calibration runs fix both before the timed sample is sized.  got (the
    GPU step's output rows, fp32 [B*H*L, d]) is compared with the oracle's
    rows of the timed sample: the step's parity at full size."""
    import oracle

    nthreads = host_threads()
    prob = oracle.Problem(w.q, w.k, w.v, w.phi, flags, alibi=alibi)
    samples = []
    for stride in (2048, 512):
        rows = _strided_rows(w, stride, 17)
        t0 = time.perf_counter()
        prob.rows(rows, nthreads)
        samples.append((rows.size, time.perf_counter() - t0))
    (n1, t1), (n2, t2) = samples
    per_row = max((t2 - t1) / max(n2 - n1, 1), 1e-9)
    fixed = max(t1 - per_row * n1, 0.0)
    want_rows = max((target_s - fixed) / per_row, n2)
    if fixed + per_row * w.batch * w.heads * w.seqlen < 2.0 * target_s:
        want_rows = w.batch * w.heads * w.seqlen
    stride = int(max(1, min(512, round(w.batch * w.heads * w.seqlen / want_rows))))
    rows = _strided_rows(w, stride, 5)
    # The calibration can misjudge the per-row cost (small samples carry the
    # thread pool's start-up), so the sample is run again until at least
    # 10 s of CPU work (or eight runs) has been timed.
    reps, dt = 0, 0.0
    while reps == 0 or (dt < min(10.0, target_s) and reps < 8):
        t0 = time.perf_counter()
        ref = prob.rows(rows, nthreads)
        dt += time.perf_counter() - t0
        reps += 1
    per = dt / reps
    i = rows % w.seqlen
    flops = float(4.0 * w.head_dim * (i + 1).sum())
    which = "every query row" if stride == 1 else f"every {stride}-th query row"
    return {"value": flops / per / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "sample": f"{rows.size} query rows ({which} of each of the {w.batch * w.heads} heads, "
                      f"with the angle scan and key/value rotation of each head), fp64, "
                      f"{reps} run(s), {dt:.1f} s in all",
            "seconds": round(per, 3), "tokens_per_s": rows.size / per,
            "parity": None if got is None else _parity(got[rows], ref,
                                                       2e-2 if w.dtype == "bf16" else 1e-4)}


def host_threads() -> int:
    """Threads for the oracle: the host's CPU share as the environment states it
    (OMP_NUM_THREADS, which the GPU hosts set to the share one GPU's jobs may
    use), else every core this process may run on."""
    aff = len(os.sched_getaffinity(0))
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        share = 0
    return min(aff, share) if share > 0 else aff


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_cpu_single_thread(target_s: float = 4.0) -> dict:
    """The oracle on one thread, on strided query rows of the small decoder
    training shape (8 x 8 heads, 1024 tokens, d=64, rotation of q and k): a
    per-core reference next to the multi-threaded baseline."""
    import oracle
    from accumulated_rotation_positional_amd import workloads as wl
    w = wl.make("train_1k")
    prob = oracle.Problem(w.q, w.k, w.v, w.phi, oracle.ROTATE_QK)
    rows = _strided_rows(w, 64, 3)
    t0 = time.perf_counter()
    prob.rows(rows, 1)
    dt = time.perf_counter() - t0
    stride = int(max(1, min(64, round(64 * dt / target_s))))
    rows = _strided_rows(w, stride, 3)
    t0 = time.perf_counter()
    prob.rows(rows, 1)
    dt = time.perf_counter() - t0
    flops = float(4.0 * w.head_dim * ((rows % w.seqlen) + 1).sum())
    return {"workload": w.name, "value": flops / dt / 1e9, "unit": "GFLOP/s", "cores": 1,
            "sample": f"{rows.size} query rows (every {stride}-th of each of the "
                      f"{w.batch * w.heads} heads, with each head's angle scan and key/value "
                      f"rotation), fp64, {dt:.1f} s", "tokens_per_s": rows.size / dt}


def _parity(got, ref, bar: float) -> dict:
    """The GPU rows against the oracle's: max |error| (the tests' bar beside
    it) and the rms error relative to the rms output."""
    err = np.abs(got.astype(np.float64) - ref)
    return {"rows": int(ref.shape[0]), "max_abs_err": float(err.max()),
            "rms_err_over_rms": float(np.sqrt((err ** 2).mean() / max((ref ** 2).mean(), 1e-300))),
            "bar_max_abs": bar, "within_bar": bool(err.max() <= bar)}


def scan_gate(binding, torch, dev, steps: int = 30) -> dict:
    """The angle scan alone on the largest workload's angle tensor (B=4, H=32,
    L=8192, 64 pairs: 268 MB in, 268 MB out, beyond the 256 MB Infinity
    Cache), where its HBM roofline is read.  Before every timed launch a
    512 MB read (a sum, which leaves only clean lines behind, so no write-back
    overlaps the scan) evicts the cache, and events bracket the scan alone.
    Seeded uniform angles: the scan's cost does not depend on the values."""
    from accumulated_rotation_positional_amd import workloads as wl
    spec = wl.SPECS["rope_8k_d128"]
    B, H, L, P = spec.batch, spec.heads, spec.seqlen, spec.head_dim // 2
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    phi = torch.rand(B, H, L, P, device=dev, generator=g) * 6.0 - 3.0
    theta = torch.empty_like(phi)
    desc = binding.make_desc(B, H, L, 2 * P, "bf16", binding.flags_for())
    state = binding.scan_state(desc, dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(10):
        binding.angle_scan(phi, desc, theta=theta, state=state)
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        flush.sum()
        e0.record(stream)
        binding.angle_scan(phi, desc, theta=theta, state=state)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
    del flush
    nbytes = 8.0 * phi.numel()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "rope_8k_d128 angles", "bound": "hbm", "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "us_per_launch": round(ms * 1e3, 2), "bytes_per_launch": nbytes}


def backward_leg(binding, torch, dev, w, q, k, v, phi, alibi, steps: int = 20) -> dict:
    """The training step's backward on the same workload: the training forward
    (which also writes the per-row log-sum-exp) once, then the backward timed
    alone (prep, dK/dV, dQ and the reverse angle scan: one C-ABI call) between
    events on its stream.  Rate: the conventional 2.5x the forward's
    algorithmic flops (the five products per causal pair: S recomputed, dP,
    dV, dK, dQ) against the bf16 matrix-core peak."""
    if w.dtype != "bf16":
        return None
    o, theta, lse, desc = binding.forward_train(q, k, v, phi, rotate_qk=True,
                                                rotate_v=w.rotate_v, alibi=alibi)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    dout = torch.randn(q.shape, device=dev, generator=g).to(torch.bfloat16)
    stream = torch.cuda.current_stream(dev)
    ws = binding.backward_workspace(desc, dev)
    for _ in range(5):
        binding.backward(desc, q, k, v, phi, theta, o, lse, dout, alibi=alibi, ws=ws)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        binding.backward(desc, q, k, v, phi, theta, o, lse, dout, alibi=alibi, ws=ws)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
    flops = 2.5 * w.flops
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": w.name, "ms": round(ms, 4), "algorithmic_flops": flops,
            "bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "outputs": "dq, dk, dv (bf16), dtheta, dphi (fp32)"}


def forget_leg(binding, torch, dev, w, q, k, v, phi, steps: int = 20) -> dict:
    """The same forward with the forget-gate bias (arp_forward_ex: scan, rotation
    pass, gate prefix pass, attention) against the same call without gates,
    each timed whole between events.  Gates log sigmoid(z), z ~ N(2, 1),
    seeded."""
    if w.dtype != "bf16":
        return None
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    z = torch.randn(w.batch, w.heads, w.seqlen, device=dev, generator=g) + 2.0
    logf = torch.nn.functional.logsigmoid(z).contiguous()
    stream = torch.cuda.current_stream(dev)

    def timed(gates):
        for _ in range(5):
            binding.forward_ex(q, k, v, phi, rotate_v=w.rotate_v, logf=gates)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for e0, e1 in evs:
            e0.record(stream)
            binding.forward_ex(q, k, v, phi, rotate_v=w.rotate_v, logf=gates)
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))

    with_g, without = timed(logf), timed(None)

    # The gated backward (arp_backward_ex: gate prefix, prep, dK/dV and dQ with
    # the gate terms and the dS sums, the two gate-gradient scans, the reverse
    # angle scan) on the gated forward's o and lse.
    o, theta, lse = binding.forward_ex(q, k, v, phi, rotate_v=w.rotate_v, logf=logf, with_lse=True)
    desc = binding.desc_for(q, binding.flags_for(rotate_v=w.rotate_v, forget=True))
    g.manual_seed(7)
    dout = torch.randn(q.shape, device=dev, generator=g).to(torch.bfloat16)
    ws = binding.backward_workspace(desc, dev)
    for _ in range(5):
        binding.backward_ex(desc, q, k, v, phi, theta, o, lse, dout, logf=logf, ws=ws)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        binding.backward_ex(desc, q, k, v, phi, theta, o, lse, dout, logf=logf, ws=ws)
        e1.record(stream)
    torch.cuda.synchronize()
    bwd = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
    # The gated kernel stops walking a row's keys once every remaining
    # probability is exactly zero, so dense causal flops over its time would
    # overstate its rate: report the two times and their ratio.
    return {"workload": w.name, "gates": "log sigmoid(z), z ~ N(2, 1)",
            "ms_with_gate": round(with_g, 4), "ms_without": round(without, 4),
            "speedup_vs_ungated": round(without / with_g, 3),
            "backward_ms_with_gate": round(bwd, 4)}


def generator_leg(binding, torch, dev, steps: int = 30) -> dict:
    """The scans that generate their step angles in the kernel, on the largest
    workload's angle shape (B=4, 32 angle heads, L=8192, 64 pairs; theta is
    268 MB): the random variant's draws (Philox), a per-token table (vocab
    256), constant frequencies.  Each writes theta only (plus 32 KB of token
    ids and the table), so the HBM roofline is on 4 bytes per element.  The
    Infinity Cache is evicted by a 512 MB read before each timed launch, as in
    the scan gate; median of the launches, each bracketed by its own events."""
    from accumulated_rotation_positional_amd import workloads as wl
    B, H, L, P = 4, 32, 8192, 64
    desc = binding.make_desc(B, H, L, 2 * P, "bf16", binding.flags_for())
    g = torch.Generator(device=dev)
    g.manual_seed(6)
    bound = torch.from_numpy(np.broadcast_to(wl.rope_frequencies(2 * P), (H, P)).copy()).to(dev)
    tokens = torch.randint(0, 256, (B, L), device=dev, generator=g, dtype=torch.int32)
    table = torch.rand(256, H, P, device=dev, generator=g) * 6.0 - 3.0
    theta = torch.empty(B, H, L, P, device=dev)
    state = binding.scan_state(desc, dev)
    calls = {
        "random": lambda i: binding.angle_scan_random(desc, 1234, i, bound, theta=theta, state=state),
        "token_table": lambda i: binding.angle_scan_tokens(desc, tokens, table, theta=theta, state=state),
        "constant": lambda i: binding.angle_scan_const(desc, bound, theta=theta),
    }
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    nbytes = 4.0 * theta.numel()
    out = {"workload": "rope_8k_d128 angles", "bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "bytes_per_launch": nbytes}
    for name, f in calls.items():
        for i in range(5):
            f(i)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for i, (e0, e1) in enumerate(evs):
            flush.sum()
            e0.record(stream)
            f(i)
            e1.record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"us_per_launch": round(ms * 1e3, 2), "achieved": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}
    # The random variant is bound by its Philox arithmetic, not by the 4 bytes
    # it writes per angle: its vector-ALU roofline, on the wave instructions
    # one launch executes (SQ_INSTS_VALU from the committed counter summary)
    # over the measured launch time, against the chip's issue rate.
    c = forward_counters("random_generator")
    if c is not None:
        rate = c["valu_insts_per_launch"] / (out["random"]["us_per_launch"] * 1e-6)
        out["random"]["alu_roofline"] = {
            "bound": "alu", "unit": "VALU wave-instr/s", "achieved": float(f"{rate:.4g}"),
            "peak": VALU_PEAK_INSTS, "frac": round(rate / VALU_PEAK_INSTS, 4),
            "valu_insts_per_launch": c["valu_insts_per_launch"],
            "valu_busy_pct_counters": c["valu_busy_pct"]}
    del flush
    return out


def decode_leg(binding, torch, dev, steps: int = 50) -> dict:
    """Decode steps at a full context: the token at the last position attends
    to every cached row.  Two cache shapes: extrap_16k's (B=2, H=8, 16384
    tokens, d=64: 67 MB of keys and values, which the 256 MB Infinity Cache
    can hold) and rope_8k_d128's (B=4, H=32, 8192 tokens, d=128: 537 MB, read
    from HBM on every step).  Per step: the append, the split-key attention and
    the combine; HBM roofline on the bytes the attention must read,
    2 * tokens * d * 2 bytes per (b, h).  The caches hold seeded random bf16
    (the cost does not depend on the values).  The same step with forget gates
    (arp_decode_step_ex, seeded log sigmoid(z) gates) is timed next to it."""
    from accumulated_rotation_positional_amd import workloads as wl
    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    for name in ("extrap_16k", "rope_8k_d128"):
        spec = wl.SPECS[name]
        B, H, L, d = spec.batch, spec.heads, spec.seqlen, spec.head_dim
        cache = binding.DecodeCache(B, H, L, d, rotate_qk=True, rotate_v=True, device=dev)
        cache.kcache.copy_(torch.randn(cache.kcache.shape, device=dev, generator=g) * d ** -0.5)
        cache.vcache.copy_(torch.randn(cache.vcache.shape, device=dev, generator=g) * d ** -0.5)
        cache.prefill()
        q, k, v = (torch.randn(B, H, d, device=dev, generator=g).to(torch.bfloat16) * d ** -0.5
                   for _ in range(3))
        phi = torch.rand(B, H, d // 2, device=dev, generator=g) * 0.5
        o = torch.empty_like(q)
        for _ in range(5):
            cache.step(L - 1, q, k, v, phi, out=o)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for e0, e1 in evs:
            e0.record(stream)
            cache.step(L - 1, q, k, v, phi, out=o)
            e1.record(stream)
        torch.cuda.synchronize()
        us = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3
        # the same step with forget gates (the gate-prefix cache adds 4 bytes per key)
        gated = binding.DecodeCache(B, H, L, d, rotate_qk=True, rotate_v=True, forget=True,
                                    device=dev)
        gated.kcache.copy_(cache.kcache)
        gated.vcache.copy_(cache.vcache)
        gated.prefill()
        logf = torch.nn.functional.logsigmoid(
            torch.randn(B, H, device=dev, generator=g) + 2.0).contiguous()
        for _ in range(5):
            gated.step(L - 1, q, k, v, phi, out=o, logf=logf)
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record(stream)
            gated.step(L - 1, q, k, v, phi, out=o, logf=logf)
            e1.record(stream)
        torch.cuda.synchronize()
        us_g = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3
        nbytes = 2.0 * L * d * 2 * B * H
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"context": L, "batch": B, "heads": H, "head_dim": d, "us_per_step": round(us, 2),
                     "tokens_per_s": round(B / (us * 1e-6), 1), "cache_bytes": nbytes,
                     "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "us_per_step_with_gate": round(us_g, 2)}
        del cache, gated
        torch.cuda.empty_cache()
    return out


def _executed(name: str, attn_ms: float) -> dict:
    """Matrix-core utilisation of the attention kernel from the flops it executes
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 per launch, committed counter summary)
    over its measured time: with a distance bias the walk skips whole tiles, so
    this, not the dense-equivalent rate, is what the matrix cores did."""
    c = forward_counters(name)
    if c is None or not c.get("attn_mfma_flops_executed"):
        return {}
    rate = c["attn_mfma_flops_executed"] / (attn_ms * 1e-3) / 1e12
    return {"attn_executed_mfma_flops": c["attn_mfma_flops_executed"],
            "attn_mfma_util": round(rate / MFMA_BF16_PEAK_TFLOPS, 4)}


def workloads_leg(binding, torch, dev, skip: str, steps: int = 20, warmup: int = 20,
                  samples: dict | None = None) -> dict:
    """The forward on every other workload, each at its full shape with seeded
    inputs.  ms_per_step: the whole forward through arp_forward (the scan with
    the key rotation fused in, then attention; fp32 I/O: scan and the fp32
    kernel), device time with the launches queued ahead; the same step
    launched kernel by kernel from Python (ms_per_step_host_launched, host
    bound on small grids) gives per-kernel event times on the stream; rates
    on the algorithmic attention flops.  Secondary figures next to the
    headline workload's.  samples (if given) receives each workload's sampled
    output rows for the parity check of the oracle leg."""
    from accumulated_rotation_positional_amd import workloads as wl
    out = {}
    for name in wl.SPECS:
        if name == skip:
            continue
        w = wl.make(name)

        def to_dev(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        q, k, v, phi = (to_dev(getattr(w, n)) for n in ("q", "k", "v", "phi"))
        alibi = to_dev(w.alibi) if w.alibi is not None else None
        flags = binding.flags_for(rotate_qk=True, rotate_v=w.rotate_v, alibi=w.use_alibi,
                                  shared_phi=w.phi_heads == 1 and w.heads != 1)
        desc = binding.desc_for(q, flags)
        ws = binding.workspace(desc, dev)
        state = binding.scan_state(desc, dev)
        theta = torch.empty_like(phi)
        o = torch.empty_like(q)
        stream = torch.cuda.current_stream(dev)
        fused = w.dtype == "f32"
        n_ev = 2 if fused else 3

        def step(evs=None):
            if evs is not None:
                evs[0].record(stream)
            binding.angle_scan(phi, desc, theta=theta, state=state)
            if evs is not None:
                evs[1].record(stream)
            if fused:
                binding.attn_fwd(q, k, v, theta, desc, alibi=alibi, out=o, ws=ws)
            else:
                binding.rotate_kv(k, v, theta, desc, ws=ws)
                if evs is not None:
                    evs[2].record(stream)
                binding.attn_rotated(q, v, theta, alibi, o, desc, ws)
            if evs is not None:
                evs[n_ev].record(stream)

        for _ in range(warmup):
            step()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev + 1)]
                  for _ in range(steps)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(steps):
            step(events[i])
        end.record(stream)
        torch.cuda.synchronize()
        ms_host = start.elapsed_time(end) / steps
        seg = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(n_ev)] for e in events])

        # The whole forward through its one entry point (arp_forward: the angle
        # scan with the key rotation fused in, then attention), one call per
        # step back to back with no events in between: on small grids the
        # kernel-by-kernel launches above are bound by the host, this one by
        # the device as long as a call's host time is below its device time.
        def forward():
            binding.forward(q, k, v, phi, rotate_v=w.rotate_v, alibi=alibi, out=o, theta=theta,
                            state=state, ws=ws)

        for _ in range(warmup):
            forward()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        f0.record(stream)
        for _ in range(steps):
            forward()
        f1.record(stream)
        torch.cuda.synchronize()
        ms_step = f0.elapsed_time(f1) / steps
        attn_ms = float(seg[:, -1].mean())
        scan_ms = float(seg[:, 0].mean())
        scan_gbs = 8.0 * w.batch * w.phi_heads * w.seqlen * (w.head_dim // 2) / (scan_ms * 1e-3) / 1e9
        attn_tf = w.flops / (attn_ms * 1e-3) / 1e12
        out[name] = {
            "shape": [w.batch, w.heads, w.seqlen, w.head_dim], "dtype": w.dtype,
            "rotate_v": w.rotate_v, "alibi": w.use_alibi, "ms_per_step": round(ms_step, 4),
            "ms_per_step_host_launched": round(ms_host, 4),
            "kernels_ms": {"angle_scan": round(scan_ms, 5),
                           "rotate_kv": round(float(seg[:, 1].mean()), 5) if n_ev == 3 else 0.0,
                           "attn_fwd": round(attn_ms, 5)},
            "tflops_step": round(w.flops / (ms_step * 1e-3) / 1e12, 2),
            "tokens_per_s": round(w.batch * w.seqlen / (ms_step * 1e-3), 1),
            **({"attn_dense_equivalent_tflops": round(attn_tf, 2)} if w.use_alibi else
               {"attn_tflops": round(attn_tf, 2),
                "attn_frac_of_bf16_peak": round(attn_tf / MFMA_BF16_PEAK_TFLOPS, 4)
                if not fused else None}),
            "scan_gbs": round(scan_gbs, 1),
            **_executed(name, attn_ms),
            "note": ("dense-equivalent: the algorithmic flops of every causal pair over the "
                     "kernel time, while the distance-bias walk skips key tiles whose "
                     "probabilities are all exactly zero; attn_mfma_util is the "
                     "matrix-core utilisation from the flops the kernel executes "
                     "(profiles/forward_counters.json)")
            if w.use_alibi else None,
        }
        if samples is not None:
            rows = _parity_rows(w)
            got = o.reshape(-1, w.head_dim)[torch.from_numpy(rows).to(dev)].float().cpu().numpy()
            samples[name] = (rows, got)
        del q, k, v, phi, alibi, ws, state, theta, o
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the path "
              "shards over (batch, head) with no exchange, so one GPU's share is the "
              "measured unit (see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch

    from accumulated_rotation_positional_amd import binding
    from accumulated_rotation_positional_amd import workloads as wl

    w = wl.make(args.workload)
    dev = torch.device("cuda:0")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v, phi = (to_dev(getattr(w, n)) for n in ("q", "k", "v", "phi"))
    alibi = to_dev(w.alibi) if w.alibi is not None else None
    flags = binding.flags_for(rotate_qk=True, rotate_v=w.rotate_v, alibi=w.use_alibi,
                              shared_phi=w.phi_heads == 1 and w.heads != 1, fused=args.fused)
    desc = binding.desc_for(q, flags)
    ws = binding.workspace(desc, dev)
    state = binding.scan_state(desc, dev)
    theta = torch.empty_like(phi)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)

    fused = args.fused or w.dtype == "f32"
    n_ev = 2

    # One step = two launches through the step entry points: the angle scan
    # with the key/value pre-rotation in its epilogue (arp_angle_scan_rotate_kv),
    # then attention with the query rotation in its prologue (arp_attn_rotated);
    # fp32 I/O or --fused: the scan, then attention rotating while it stages.
    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        if fused:
            binding.angle_scan(phi, desc, theta=theta, state=state)
        else:
            binding.angle_scan_rotate_kv(phi, k, v, desc, theta=theta, state=state, ws=ws)
        if evs is not None:
            evs[1].record(stream)
        if fused:
            binding.attn_fwd(q, k, v, theta, desc, alibi=alibi, out=o, ws=ws)
        else:
            binding.attn_rotated(q, v, theta, alibi, o, desc, ws)
        if evs is not None:
            evs[2].record(stream)

    # Clock warm-up: an idle GPU starts below the clock it holds under a long
    # matrix-core load (the attention kernel reads ~15% slower over the first
    # few steps).  Whole steps are run for a fixed wall time, untimed and
    # reported as their own field; the --warmup steps and the timed --steps
    # steps follow unchanged.
    warm_steps, t_warm = 0, time.perf_counter()
    while time.perf_counter() - t_warm < args.clock_warmup_s:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        warm_steps += 20
    t_warm = time.perf_counter() - t_warm
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # The timed region holds exactly the K steps, bracketed by device
    # synchronisation; events between the kernels of each step give the
    # per-kernel durations on the stream the kernels run on.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev + 1)]
              for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        step(events[s])
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(end) / args.steps
    seg = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(n_ev)] for e in events])
    scan_ms = float(seg[:, 0].mean())
    attn_ms = float(seg[:, -1].mean())

    flops = w.flops
    tflops = flops / (ms_step * 1e-3) / 1e12
    tokens = w.batch * w.seqlen / (ms_step * 1e-3)
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    # algorithmic bytes of the first launch: phi read and theta written (4 + 4
    # bytes per token and pair of each angle stream); fused with the key
    # rotation also k read and k~ written (2 + 2 bytes per element), and v /
    # v~ likewise with value transport
    scan_bytes = 8.0 * w.batch * w.phi_heads * w.seqlen * (w.head_dim // 2)
    if not fused:
        scan_bytes += 4.0 * w.batch * w.heads * w.seqlen * w.head_dim * (2 if w.rotate_v else 1)
    scan_gbs = scan_bytes / (scan_ms * 1e-3) / 1e9
    traffic, scan_traffic = measured_traffic(w.name)
    if fused:
        traffic = None

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "tokens_per_s": round(tokens, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_warmup": {"seconds": round(t_warm, 3), "steps": warm_steps,
                         "note": "untimed whole steps before the --warmup steps"},
        "ms_per_step": round(ms_step, 4),
        "wall_s_timed": round(t_wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; learned-angle generator phi = W x)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.seqlen,
                   "head_dim": w.head_dim, "rotate_v": w.rotate_v, "alibi": w.use_alibi,
                   "rotation": "fused-in-staging" if fused else "pre-rotation pass"},
        "kernels_ms": {("angle_scan" if fused else "angle_scan_rotate_kv"): round(scan_ms, 5),
                       "attn_fwd": round(attn_ms, 5)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic},
        "scan_roofline": {"kernel": "angle_scan" if fused else "angle_scan_rotate_kv",
                          "bound": "hbm", "achieved": round(scan_gbs, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(scan_gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_launch": scan_bytes, "traffic": scan_traffic},
    }
    if not args.forward_only:
        result["scan_hbm_gate"] = scan_gate(binding, torch, dev)
        result["angle_generators"] = generator_leg(binding, torch, dev)
    wl_samples = {}
    if not args.fused and not args.forward_only:
        result["backward"] = backward_leg(binding, torch, dev, w, q, k, v, phi, alibi)
        result["decode"] = decode_leg(binding, torch, dev)
        result["forget_gate"] = forget_leg(binding, torch, dev, w, q, k, v, phi)
        if not args.no_workloads:
            result["workloads"] = workloads_leg(binding, torch, dev, w.name, samples=wl_samples)
    if not args.no_cpu_baseline:
        import oracle
        of = (oracle.ROTATE_QK | (oracle.ROTATE_V if w.rotate_v else 0) |
              (oracle.ALIBI if w.use_alibi else 0))
        got = o.float().cpu().numpy().reshape(-1, w.head_dim)
        result["cpu_baseline"] = run_cpu_baseline(w, of, w.alibi, args.cpu_seconds, got)
        result["cpu_baseline"]["single_thread"] = run_cpu_single_thread()
        if wl_samples:
            result["cpu_baseline"]["parity_per_workload"] = run_workload_parity(wl_samples)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
