"""Benchmark: fused 1-bit compress + frozen-v update on one MI355X.

Headline (one JSON line on stdout): params/s of onebit_compress_update on the
BERT-Large-shaped flat vector (335,143,938 fp32 params in 393 tensors, one scale
per tensor, 8 masked tensors, one compressed step per call), with inputs
resident in HBM.  A "step" is one such call.  Also reported:
  roofline     the dominant kernel (the one-pass persistent compression kernel):
               algorithmic bytes per launch / its mean launch time from HIP events
               recorded around each launch on the launch stream, against 8 TB/s;
  cpu_baseline the CPU oracle (single thread) on a bounded sample of the same
               workload, timed on this host;
  ceiling      a plain streaming kernel with the same 5-read/3-write mix, timed
               now on this device, and the one-pass kernel's fraction of it;
  rows         the other hot-path kernels measured the same way (warmup Adam step,
               the GPT-2-XL-shaped bf16-gradient vector, the 16-worker simulated
               all-reduce, QSDP quantize/dequantize) unless --headline-only.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only]

Profiling (rocprofv3 runs the program itself, so these modes only do the work):
  python bench.py --profile            headline workload, a few steps, then a
                                       1 GiB device-to-device copy used to
                                       calibrate the FETCH_SIZE/WRITE_SIZE counters
  python bench.py --profile-allreduce  the same for the 16-worker simulated all-reduce
  python bench.py --summarize-allreduce KT FETCH WRITE SQ
  python bench.py --summarize-profile KT FETCH WRITE
                                       turn three rocprofv3 CSV output directories
                                       (kernel trace+stats, --pmc FETCH_SIZE,
                                       --pmc WRITE_SIZE) into the text summary kept
                                       under profiles/ (printed to stdout)
  python bench.py --placement          LoCo and an in-place stream by buffer placement
  python bench.py --ceilings [--ceilings-elems N]
                                       streaming ceilings by read/write mix, cache
                                       policy and workgroup shape, N fp32 elements
                                       per stream (default 2^28; markdown on stdout)
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
B_COMPRESS_F32 = 32.125      # read g,m,e,v,x (20 B); write m,e,x (12 B); bits (1/8 B)
B_COMPRESS_BF16_COPY = 32.125  # read g bf16 (2),m,e,v,x (16); write m,e,x (12), x_bf16 (2); bits
B_WARMUP = 28.0              # read g,m,v,x; write m,v,x
B_COMPRESS_PACKED = 24.25    # read g,e,v,x (16 B) and 1/8 B of momentum words; write e,x (8 B), bits
B_WORKER = 16.125            # read g,m,e; write e; bits
B_WORKER_F16 = 14.125        # read g fp16 (2), m, e; write e; bits
B_FINISH_MASK = 21.0         # read m, mask (1), v, x; write m, x
B_FINISH_PACKED = 13.125     # read 1/8 B of server words, mask (1), v, x; write x
B_QSDP4, B_QSDP8 = 2.0 + 0.5 + 8.0 / 1024, 2.0 + 1.0 + 8.0 / 1024
B_QSDP_STAT = 22.0           # the statistic: read x bf16 (2), y fp32 (4), ysum fp64 (8); write ysum (8)
B_QSDP_MAE = 10.0            # mean abs error of the seed average: read x bf16 (2), ysum fp64 (8)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def ensure_built():
    from error_compensated_bit_amd import onebit
    if not os.path.exists(onebit.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    onebit.load()


class KernelTimer:
    """Per-kernel-class HIP event timing over a region (library launch profiler);
    classes: the kernel classes to bracket with events (None: all)."""

    def __init__(self, classes=None):
        self.classes = classes

    def __enter__(self):
        from error_compensated_bit_amd import onebit as ob
        ob.onebit_profile_begin(self.classes)
        return self

    def __exit__(self, *exc):
        from error_compensated_bit_amd import onebit as ob
        self.result = ob.onebit_profile_end()
        return False

    def mean_ms(self, cls):
        ms, n = self.result[cls]
        return ms / n if n else None


def timed(fn, steps, warmup, classes=()):
    """Seconds per call over `steps` timed calls after `warmup` untimed ones, and the
    library's per-kernel event times.  Each HIP event adds a few microseconds between
    launches, so the timed calls carry events only around the kernel classes named in
    `classes` (kt.timed); kt itself times every kernel class in a separate pass of up
    to 10 calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    with KernelTimer(classes) as kt_timed:
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    with KernelTimer() as kt:
        for _ in range(min(steps, 10)):
            fn()
        torch.cuda.synchronize()
    kt.timed = kt_timed
    return (t1 - t0) / steps, kt


def compress_setup(wl, dev):
    import torch
    from error_compensated_bit_amd import onebit as ob
    from error_compensated_bit_amd import workloads as W
    x, m, e, v = W.init_state(wl, device=dev)
    g = W.gradient(wl, 1, device=dev)
    plan = ob.onebit_plan_create(wl.chunk_off, wl.tensor_off, wl.tensor_keep)
    bits = torch.zeros(ob.onebit_plan_words(plan), dtype=torch.int32, device=dev)
    scales = torch.zeros(ob.onebit_plan_chunks(plan), dtype=torch.float32, device=dev)
    ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=dev)
    xb = torch.zeros(wl.n, dtype=torch.bfloat16, device=dev) if wl.x_bf16_copy else None
    hp = dict(lr=wl.hyper["lr"], beta1=wl.hyper["beta1"], eps=wl.hyper["eps"], weight_decay=wl.hyper["weight_decay"])

    def step():
        ob.onebit_compress_update(plan, g, m, e, v, x, xb, bits, scales, workspace=ws, **hp)

    return plan, step, ws


def onepass_elements(wl, plan):
    """Elements of the chunks the one-pass kernel handles: a chunk goes there when
    its tiles fit the resident pipeline, i.e. it has at most
    onebit_onepass_max_elements() elements."""
    import numpy as np
    from error_compensated_bit_amd import onebit as ob
    lens = np.diff(wl.chunk_off)
    return int(lens[lens <= ob.onebit_onepass_max_elements()].sum())


def bench_compress(wl, steps, warmup, dev, bpe):
    """The timed steps carry HIP events around the one-pass launches only; the
    breakdown over every kernel of the step comes from timed()'s separate pass."""
    from error_compensated_bit_amd import onebit as ob
    plan, step, ws = compress_setup(wl, dev)
    t, kt = timed(step, steps, warmup, classes=("compress_onepass",))
    assert ob.onebit_workspace_status(ws) == 0, "a cross-workgroup wait timed out"
    n1 = onepass_elements(wl, plan)
    k_ms = kt.timed.mean_ms("compress_onepass")
    res = dict(seconds_per_call=t, params_per_s=wl.n / t, gbps=bpe * wl.n / t / 1e9,
               onepass_elements=n1, onepass_ms=k_ms, plan=ob.onebit_plan_stats(plan),
               kernels={k: v for k, v in kt.result.items() if v[1]})
    if k_ms:
        res["onepass_gbps"] = bpe * n1 / (k_ms * 1e-3) / 1e9
    return res


def host_cpu():
    """(CPU model name from /proc/cpuinfo, logical CPUs of the host, CPUs this process may use)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = sorted(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = list(range(os.cpu_count() or 1))
    return model, os.cpu_count(), allowed


class pinned_to_one_core:
    """Run the enclosed block with this thread bound to one allowed CPU (the last
    one), restoring the previous affinity afterwards."""

    def __enter__(self):
        self.core = None
        try:
            self.prev = os.sched_getaffinity(0)
            self.core = max(self.prev)
            os.sched_setaffinity(0, {self.core})
        except (AttributeError, OSError):
            self.prev = None
        return self

    def __exit__(self, *exc):
        if self.prev is not None:
            os.sched_setaffinity(0, self.prev)
        return False


def cpu_baseline(wl, dev, budget_s=12.0):
    """Time the CPU oracle on whole chunks of the workload (successive compressed
    steps over the vector, chunk by chunk) until about budget_s of CPU work, with the
    timing thread pinned to one core."""
    import numpy as np
    import oracle
    from error_compensated_bit_amd import workloads as W
    state = [t.cpu().numpy() for t in W.init_state(wl, device=dev)]       # x, m, e, v
    g = W.gradient(wl, 1, device=dev)
    g = (g.float() if wl.grad_bf16 else g).cpu().numpy()
    model, ncpu, allowed = host_cpu()
    with pinned_to_one_core() as pin:
        done, spent, calls, steps = _cpu_baseline_loop(wl, state, g, budget_s)
    return dict(value=done / spent, unit="params/s", cores=1, kind="oracle",
                sample=f"{calls} whole-chunk calls over {steps} compressed step(s) of the same workload "
                       f"({done} params), single-threaded C oracle, in place on host copies",
                seconds=spent, cpu_model=model, host_cpus=ncpu, cpus_allowed=len(allowed), pinned_core=pin.core)


def _cpu_baseline_loop(wl, state, g, budget_s):
    import numpy as np
    import oracle
    done = 0
    spent = 0.0
    calls = 0
    steps = 0
    while spent < budget_s:
        steps += 1
        for j in range(wl.n_chunks):
            lo, hi = int(wl.chunk_off[j]), int(wl.chunk_off[j + 1])
            off = np.array([0, hi - lo], np.int64)
            t_off = t_keep = None
            if wl.tensor_keep is not None:
                t = int(np.searchsorted(wl.tensor_off, lo, side="right") - 1)
                t_off, t_keep = np.array([0, hi - lo], np.int64), wl.tensor_keep[t:t + 1]
            x, m, e, v = (a[lo:hi] for a in state)
            gj = g[lo:hi]
            t0 = time.perf_counter()
            oracle.compress_update(off, gj, m, e, v, x, tensor_off=t_off, tensor_keep=t_keep, lr=1e-3, beta1=0.9,
                                   eps=1e-8)
            spent += time.perf_counter() - t0
            done += hi - lo
            calls += 1
            if spent >= budget_s:
                break
    return done, spent, calls, steps


def _oracle_rate(call, units, budget_s):
    """Repeat call() until budget_s of CPU time is spent; units processed per second."""
    spent, calls = 0.0, 0
    while spent < budget_s or calls == 0:
        t0 = time.perf_counter()
        call()
        spent += time.perf_counter() - t0
        calls += 1
    return units * calls / spent, calls


def cpu_row_baselines(rows, budget_s=1.0):
    """The CPU oracle timed beside each secondary row, on a bounded seeded sample of
    that row's workload (same dtypes, distributions and bucket or chunk sizes, fewer
    elements); single-threaded, in place on host arrays.  Step rows are scaled from
    the sample to the row's full size."""
    import numpy as np
    import torch
    import oracle
    from error_compensated_bit_amd import workloads as W

    rng = np.random.default_rng(4242)

    def put(key, value, unit, sample, calls):
        if key in rows:
            rows[key]["cpu_oracle"] = dict(value=value, unit=unit, cores=1, kind="oracle",
                                           sample=f"{sample}; {calls} call(s)")

    # warmup Adam
    n = 1 << 22
    x, m, v = (rng.standard_normal(n) * 0.02).astype(np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    r, c = _oracle_rate(lambda: oracle.adam_warmup_step(x, m, v, g, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                                                        weight_decay=0.0, bias_correction=False, step=1), n, budget_s)
    put("warmup_adam_bert_large", r, "params/s", f"{n} fp32 params", c)

    # QSDP: bf16 weights N(0, 0.02), buckets of 1024
    q = W.QsdpWorkload()
    n = 1 << 21
    xq = (torch.from_numpy(rng.standard_normal(n).astype(np.float32)) * q.std).to(torch.bfloat16)
    xb = xq.view(torch.int16).numpy().view(np.uint16)
    for bits in (4, 8):
        r, c = _oracle_rate(lambda: oracle.qsdp_quantize(xb, bucket=q.bucket, bits=bits, seed=0), n, budget_s)
        put(f"qsdp{bits}_quantize", r, "elems/s", f"{n} bf16 weights, buckets of {q.bucket}", c)
        codes, bmin, bmax = oracle.qsdp_quantize(xb, bucket=q.bucket, bits=bits, seed=0)
        r, c = _oracle_rate(lambda: oracle.qsdp_dequantize(codes, bmin, bmax, n, bucket=q.bucket, bits=bits), n,
                            budget_s)
        put(f"qsdp{bits}_dequantize", r, "elems/s", f"{n} bf16 weights, buckets of {q.bucket}", c)

    # one seed of the 64-seed statistic: oracle quantize, dequantize to fp32, fp64 sums
    xf = oracle.bf16_bits_to_f32(xb).astype(np.float64)

    def stat_seed():
        cds, mn_, mx_ = oracle.qsdp_quantize(xb, bucket=q.bucket, bits=4, seed=1)
        _, yf = oracle.qsdp_dequantize(cds, mn_, mx_, n, bucket=q.bucket, bits=4, want_f32=True)
        d = yf.astype(np.float64) - xf
        return d.sum(), (d * d).sum()
    r, c = _oracle_rate(stat_seed, n, budget_s)
    put("qsdp4_seed_statistic", r, "elems/s", f"one seed over {n} bf16 weights (oracle draws, numpy fp64 sums)", c)

    # QSGD / LoCo on bf16 gradients with per-block scales
    qg = W.QsgdWorkload()
    n = 1 << 20
    gw = [W.qsgd_gradient(qg, w, device="cpu", n=n).view(torch.int16).numpy().view(np.uint16) for w in range(qg.W)]
    for bits in (4, 8):
        r, c = _oracle_rate(lambda: oracle.qsgd_quantize(gw[0], bucket=qg.bucket, bits=bits, seed=7), n, budget_s)
        put(f"qsgd{bits}_quantize", r, "elems/s", f"{n} bf16 gradient elements, buckets of {qg.bucket}", c)
        enc = [oracle.qsgd_quantize(gw[w], bucket=qg.bucket, bits=bits, seed=100 + w) for w in range(qg.W)]
        codes = np.stack([e_[0] for e_ in enc])
        norms = np.stack([e_[1] for e_ in enc])
        r, c = _oracle_rate(lambda: oracle.qsgd_reduce(codes, norms, n, bucket=qg.bucket, bits=bits), n, budget_s)
        put(f"qsgd{bits}_reduce_{qg.W}x{qg.shard}", r, "elems/s",
            f"{qg.W} workers' streams over a {n}-element shard", c)
    err = np.zeros(n, np.float32)
    g32 = oracle.bf16_bits_to_f32(gw[0])
    r, c = _oracle_rate(lambda: oracle.loco_quantize(g32, err, bucket=qg.bucket, bits=4, beta=0.9, seed=7), n,
                        budget_s)
    put("loco4_quantize", r, "elems/s", f"{n} gradient elements, buckets of {qg.bucket}", c)

    # the simulated all-reduce and full step: one chunk of the sample per worker
    a = W.AllreduceWorkload()
    n = 1 << 20
    off = np.array([0, n], np.int64)
    gs = [(rng.standard_normal(n) * a.grad_std).astype(np.float32) for _ in range(a.W)]
    g16 = [gg.astype(np.float16) for gg in gs]
    ms = np.zeros(n, np.float32)
    es = [np.zeros(n, np.float32) for _ in range(a.W)]
    e_s = np.zeros(n, np.float32)
    vv = (rng.uniform(0.5, 2.0, n) * 1e-6).astype(np.float32)
    xx = (rng.standard_normal(n) * 0.02).astype(np.float32)
    mask = (rng.random(n) < 0.98).astype(np.uint8)

    def exchange(grads, finish):
        enc = [oracle.compress_update(off, grads[w], ms, es[w], beta1=0.9) for w in range(a.W)]
        wb = np.stack([e_[0] for e_ in enc])
        wsc = np.stack([e_[1] for e_ in enc])
        _, _, mo = oracle.server_reduce(off, wb, wsc, e_s)
        if finish:
            oracle.momentum_update(mo, vv, xx, mask=mask, lr=1e-3, eps=1e-8, weight_decay=0.01)

    scale = a.n / n * 1e3
    for key, grads, fin in (("allreduce_16x64M", gs, False), ("full_step_16x64M_f16_mask", g16, True),
                            ("full_step_16x64M_f16_mask_packed_m", g16, True),
                            ("driver_workers_16x64M_f16_mask_packed_m", g16, True)):
        r, c = _oracle_rate(lambda: exchange(grads, fin), 1.0, budget_s)
        put(key, scale / r, "ms_per_step", f"{a.W} workers over a {n}-element sample, time scaled by {a.n // n}", c)

    shard = n // a.W
    soff = np.array([0, shard], np.int64)

    def share_timed():
        # the workers' shard encodings stand in for data received from peers: not timed
        wb, wsc, _ = oracle.compress_update(off, g16[0], ms, es[0], beta1=0.9)
        oracle.server_reduce(soff, shard_bits, shard_scales, e_s[:shard], want_m=True)
        oracle.momentum_update(oracle.decompress(off, wb, wsc), vv, xx, mask=mask, lr=1e-3, eps=1e-8,
                               weight_decay=0.01)
    sw = (shard + 31) // 32
    enc = [oracle.compress_update(soff, g16[w][:shard], ms[:shard].copy(), es[w][:shard], beta1=0.9)
           for w in range(a.W)]
    shard_bits = np.stack([e_[0][:sw] for e_ in enc])
    shard_scales = np.stack([e_[1] for e_ in enc])
    r, c = _oracle_rate(share_timed, 1.0, budget_s)
    for key in ("gpu_share_of_16_64M_f16_mask", "gpu_share_of_16_64M_f16_mask_packed_m"):
        put(key, scale / r, "ms_per_step", f"own worker and finish over a {n}-element sample, server over "
                                          f"{shard} elements of 16 workers, time scaled by {a.n // n}", c)

    # packed momentum (the oracle decompresses the previous words into m) and GPT-2-XL chunks
    n = 1 << 21
    off2 = np.array([0, n // 2, n], np.int64)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m, e = np.zeros(n, np.float32), np.zeros(n, np.float32)
    v = (rng.uniform(0.5, 2.0, n) * 1e-6).astype(np.float32)
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    pb, psc, _ = oracle.compress_update(off2, g, m, e, v, x, lr=1e-3, beta1=0.9, eps=1e-8)

    def packed():
        mm = oracle.decompress(off2, pb, psc)
        oracle.compress_update(off2, g, mm, e, v, x, lr=1e-3, beta1=0.9, eps=1e-8)
    r, c = _oracle_rate(packed, n, budget_s)
    put("compress_bert_large_packed_m", r, "params/s", f"two chunks of {n // 2} fp32 params", c)
    gb = oracle.f32_to_bf16_bits(g)
    r, c = _oracle_rate(lambda: oracle.compress_update(off2, gb, m, e, v, x, lr=1e-3, beta1=0.9, eps=1e-8,
                                                       want_bf16=True), n, budget_s)
    put("compress_gpt2_xl_bf16", r, "params/s", f"two chunks of {n // 2} params, bf16 g, bf16 copy of x", c)


PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "compress_onepass_bert_large.md")
ONEPASS_SOURCE = os.path.join(ROOT, "error_compensated_bit_amd", "csrc", "compress.hip")
CALIBRATION_FLOATS = 1 << 28          # 1 GiB copied by the profile mode


# What the profiled one-pass kernel and its launch are built from: its source, the
# headers it includes, the plan code that lays out its tiles, and the build flags.
DIGEST_FILES = ("csrc/compress.hip", "csrc/device_common.h", "csrc/internal.h", "csrc/plan.hip", "build.py")


def _code_text(path):
    """A source file without its comments and with runs of whitespace collapsed, so
    that the digests below change with the code and not with its commentary."""
    import re
    with open(path, encoding="utf-8") as f:
        text = f.read()
    if path.endswith(".py"):
        text = re.sub(r"#[^\n]*", "", text)
    else:
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
    return " ".join(text.split()).encode()


def source_digest():
    h = hashlib.sha256()
    for rel in DIGEST_FILES:
        h.update(_code_text(os.path.join(ROOT, "error_compensated_bit_amd", rel)))
    return h.hexdigest()[:16]


def profile_mode(steps):
    """Work for rocprofv3: the headline step `steps` times, then a plain 1 GiB copy."""
    import torch
    ensure_built()
    from error_compensated_bit_amd import workloads as W
    dev = "cuda:0"
    wl = W.bert_like()
    plan, step, ws = compress_setup(wl, dev)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    src = torch.ones(CALIBRATION_FLOATS, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)        # plain streaming copy: 16-byte vector loads and stores
    torch.cuda.synchronize()
    log(f"[profile] {steps} steps of {wl.name} and one {CALIBRATION_FLOATS * 4} B copy done")


QUANT_SUMMARY = os.path.join(ROOT, "profiles", "quantizers_valu.md")
QUANT_FILES = ("csrc/qsdp.hip", "csrc/qsgd.hip", "csrc/quant_common.h", "csrc/device_common.h", "build.py")
VALU_LANE_OPS_PER_S = 256 * 64 * 2.4e9     # 256 CUs x 64 lanes (4 SIMD16, one wave64 op per 4 clocks) x 2.4 GHz


def quant_digest():
    h = hashlib.sha256()
    for rel in QUANT_FILES:
        h.update(_code_text(os.path.join(ROOT, "error_compensated_bit_amd", rel)))
    return h.hexdigest()[:16]


def quantizer_calls(dev):
    """(kernel-name fragment, label, elements, call) for the ALU-bound quantizers at full size."""
    import torch
    from error_compensated_bit_amd import onebit as ob
    from error_compensated_bit_amd import workloads as W
    q = W.QsdpWorkload()
    xq = W.qsdp_weights(q, device=dev)
    gq = W.qsgd_gradient(W.QsgdWorkload(), 0, device=dev)
    nb = (q.n + q.bucket - 1) // q.bucket
    codes = torch.zeros(q.n, dtype=torch.uint8, device=dev)
    f1, f2 = torch.zeros(nb, device=dev), torch.zeros(nb, device=dev)
    err = torch.zeros(q.n, device=dev)
    return [
        ("k_qsdp_quantize_1024<4>", "qsdp4_quantize", q.n, lambda: ob.qsdp_quantize(xq, q.bucket, 4, 0, codes, f1, f2)),
        ("k_qsdp_quantize_1024<8>", "qsdp8_quantize", q.n, lambda: ob.qsdp_quantize(xq, q.bucket, 8, 0, codes, f1, f2)),
        ("k_qsgd_quantize_1024<4, 1, false, false>", "qsgd4_quantize", q.n,
         lambda: ob.qsgd_quantize(gq, q.bucket, 4, 0, codes, f1)),
        ("k_qsgd_quantize_1024<8, 1, false, false>", "qsgd8_quantize", q.n,
         lambda: ob.qsgd_quantize(gq, q.bucket, 8, 0, codes, f1)),
        ("k_qsgd_quantize_1024<4, 1, true, false>", "loco4_quantize", q.n,
         lambda: ob.loco_quantize(gq, err, q.bucket, 4, 0.9, 0, codes, f1)),
    ]


def profile_quantizers():
    """Work for rocprofv3: each ALU-bound quantizer twice at full size."""
    import torch
    ensure_built()
    for _, label, _, call in quantizer_calls("cuda:0"):
        call()
        call()
        torch.cuda.synchronize()
        log(f"[profile] {label} done")


def summarize_quantizers(kt_dir, pmc_dir):
    """VALU instructions per element of each quantizer and its issue-rate bound."""
    import numpy as np
    stats = {_short(r["Name"]): r for r in _rows(kt_dir, "kernel_stats.csv")}
    valu = {}
    for r in _rows(pmc_dir, "counter_collection.csv"):
        if r.get("Counter_Name") == "SQ_INSTS_VALU":
            valu.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    out = ["# ALU-bound quantizers: VALU instructions per element and issue-rate bound", ""]
    out.append("Commands (from the repository root, on one MI355X):")
    out.append("```")
    out.append(f"rocprofv3 --kernel-trace --stats --output-format csv -d {kt_dir} -o bench -- python3 bench.py "
               f"--profile-quantizers")
    out.append(f"rocprofv3 --pmc SQ_INSTS_VALU --output-format csv -d {pmc_dir} -o bench -- python3 bench.py "
               f"--profile-quantizers")
    out.append(f"python bench.py --summarize-quantizers {kt_dir} {pmc_dir}")
    out.append("```")
    out.append(f"Quantizer source digest: {quant_digest()}")
    out.append("")
    out.append(f"Issue-rate bound: {VALU_LANE_OPS_PER_S / 1e12:.2f} T VALU lane-instructions/s (256 CUs x 4 SIMD16 x "
               f"one wave64 instruction per 4 clocks x 2.4 GHz); elements/s bound = that / (SQ_INSTS_VALU x 64 / "
               f"elements).  Transcendental and fp64 instructions issue at lower rates, so the bound is optimistic.  "
               f"The QSGD rows are the whole-bucket kernel; the one-workgroup launch for the ragged last bucket "
               f"(256 elements) is not counted.")
    out.append("")
    out.append("| kernel | elements | average ns | SQ_INSTS_VALU per dispatch | VALU lane-instr per element | "
               "bound G elem/s | achieved G elem/s | fraction |")
    out.append("|---|---|---|---|---|---|---|---|")
    for frag, label, n, _ in quantizer_calls_meta():
        key = next((k for k in stats if frag in k), None)
        vkey = next((k for k in valu if frag in k), None)
        if key is None or vkey is None:
            continue
        ns = float(stats[key]["AverageNs"])
        per_elem = float(np.median(valu[vkey])) * 64.0 / n
        bound = VALU_LANE_OPS_PER_S / per_elem
        ach = n / (ns * 1e-9)
        out.append(f"| {label} | {n} | {ns:.0f} | {np.median(valu[vkey]):.0f} | {per_elem:.2f} | {bound / 1e9:.0f} | "
                   f"{ach / 1e9:.0f} | {ach / bound:.3f} |")
        out.append(f"<!-- {label} valu_lane_instr_per_element={per_elem:.4f} -->")
    return "\n".join(out) + "\n"


def quantizer_calls_meta():
    n = 1_300_000_000
    return [("k_qsdp_quantize_1024<4>", "qsdp4_quantize", n, None), ("k_qsdp_quantize_1024<8>", "qsdp8_quantize", n, None),
            ("k_qsgd_quantize_1024<4, 1, false, false>", "qsgd4_quantize", n, None),
            ("k_qsgd_quantize_1024<8, 1, false, false>", "qsgd8_quantize", n, None),
            ("k_qsgd_quantize_1024<4, 1, true, false>", "loco4_quantize", n, None)]


def summarize_kernels(kt_dir, command):
    """Markdown table of the library's kernels in a kernel-trace + stats run."""
    stats = _rows(kt_dir, "kernel_stats.csv")
    out = ["# Kernel times of a whole benchmark run (rocprofv3 --kernel-trace --stats)", ""]
    out.append("Commands (from the repository root, on one MI355X):")
    out.append("```")
    out.append(f"rocprofv3 --kernel-trace --stats --output-format csv -d {kt_dir} -o bench -- python3 {command}")
    out.append(f"python bench.py --summarize-kernels {kt_dir} '{command}'")
    out.append("```")
    out.append(f"Library source digest: {source_digest()}; quantizer source digest: {quant_digest()}")
    out.append("")
    out.append("| kernel | calls | average ns | min ns | max ns | share of GPU time |")
    out.append("|---|---|---|---|---|---|")
    for r in stats:
        if "onebit::" in r["Name"]:
            out.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                       f"{r['MaxNs']} | {float(r['Percentage']):.2f}% |")
    return "\n".join(out) + "\n"


def valu_per_element():
    """{label: VALU lane-instructions per element} from the committed summary, if the sources match."""
    try:
        text = open(QUANT_SUMMARY).read()
    except OSError:
        return {}
    if f"Quantizer source digest: {quant_digest()}" not in text:
        return {}
    res = {}
    for line in text.splitlines():
        if line.startswith("<!-- ") and "valu_lane_instr_per_element=" in line:
            label, kv = line[5:-4].split(" ", 1)
            res[label] = float(kv.split("=")[1])
    return res


def _rows(dirname, suffix):
    files = glob.glob(os.path.join(dirname, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {dirname}")
    with open(files[0], newline="") as f:
        return list(csv.DictReader(f))


def profile_allreduce(steps):
    """Work for rocprofv3: `steps` simulated all-reduce steps (16 workers x 64M), then a plain 1 GiB copy."""
    import torch
    ensure_built()
    from error_compensated_bit_amd import onebit as ob
    from error_compensated_bit_amd import workloads as W
    dev = "cuda:0"
    a = W.AllreduceWorkload()
    plan = ob.onebit_plan_create(a.chunk_off)
    words, nch = ob.onebit_plan_words(plan), ob.onebit_plan_chunks(plan)
    m = torch.zeros(a.n, device=dev)
    e = torch.zeros((a.W, a.n), device=dev)
    es = torch.zeros(a.n, device=dev)
    grads = torch.randn((a.W, a.n), device=dev) * a.grad_std
    wbits = torch.zeros((a.W, words), dtype=torch.int32, device=dev)
    wsc = torch.zeros((a.W, nch), device=dev)
    sbits = torch.zeros(words, dtype=torch.int32, device=dev)
    ssc = torch.zeros(nch, device=dev)
    wsp = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=dev)
    for _ in range(steps):
        for w in range(a.W):
            ob.onebit_compress_update(plan, grads[w], m, e[w], None, None, None, wbits[w], wsc[w], lr=0.0,
                                      beta1=0.9, eps=1e-8, weight_decay=0.0, workspace=wsp)
        ob.onebit_server_reduce(plan, wbits, wsc, es, sbits, ssc, m, wsp)
    torch.cuda.synchronize()
    assert ob.onebit_workspace_status(wsp) == 0, "a cross-workgroup wait timed out"
    del e, grads
    src = torch.ones(CALIBRATION_FLOATS, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"[profile] {steps} all-reduce steps of {a.W} x {a.n} and one {CALIBRATION_FLOATS * 4} B copy done")


ALLREDUCE_SUMMARY = os.path.join(ROOT, "profiles", "allreduce_worker_server_16x64M.md")
SQ_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
               "SQ_INSTS_SALU")


def summarize_allreduce(kt_dir, fetch_dir, write_dir, sq_dir=None):
    """Kernel time, HBM traffic and (with sq_dir) issue counters of the worker
    (compress-only) and server launches."""
    import numpy as np
    from error_compensated_bit_amd import workloads as W
    a = W.AllreduceWorkload()
    stats = {_short(r["Name"]): r for r in _rows(kt_dir, "kernel_stats.csv")}
    per = {}
    dirs = [("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)]
    if sq_dir:
        dirs += [(k, sq_dir) for k in SQ_COUNTERS]
    for key, d in dirs:
        for r in _rows(d, "counter_collection.csv"):
            if r.get("Counter_Name") == key:
                per.setdefault((key, _short(r["Kernel_Name"])), []).append(float(r["Counter_Value"]))
    def counter(key, frag, how=np.median):
        vals = [v for (k, name), vs in per.items() if k == key and frag in name for v in vs]
        return float(how(vals)) if vals else None
    cal = CALIBRATION_FLOATS * 4
    f_scale = cal / (counter("FETCH_SIZE", "neg_kernel", np.max) * 1024.0)
    w_scale = cal / (counter("WRITE_SIZE", "neg_kernel", np.max) * 1024.0)
    out = [f"# Worker and server launches of the simulated all-reduce ({a.W} workers x {a.n} fp32, "
           f"{len(a.chunk_off) - 1} chunks)", ""]
    out.append("Commands (from the repository root, on one MI355X):")
    out.append("```")
    runs = [(kt_dir, "--kernel-trace --stats"), (fetch_dir, "--pmc FETCH_SIZE"), (write_dir, "--pmc WRITE_SIZE")]
    if sq_dir:
        runs.append((sq_dir, "--pmc " + " ".join(SQ_COUNTERS)))
    for d, extra in runs:
        out.append(f"rocprofv3 {extra} --output-format csv -d {d} -o bench -- python3 bench.py --profile-allreduce")
    out.append(f"python bench.py --summarize-allreduce {kt_dir} {fetch_dir} {write_dir}" + (f" {sq_dir}" if sq_dir else ""))
    out.append("```")
    out.append(f"Library source digest: {source_digest()}")
    out.append("")
    out.append(f"Counter scale from the plain {cal} B copy: FETCH_SIZE x{f_scale:.4f}, WRITE_SIZE x{w_scale:.4f}.  "
               f"Algorithmic bytes per element: worker 16.125 (read g, m, e; write e, sign bits), server "
               f"{a.W / 8 + 12.125:.3f} (read {a.W} workers' sign bits and the server error; write the server "
               f"error, the decompressed momentum and the server's sign bits).")
    out.append("")
    out.append("| launch | calls | average ns | read bytes | written bytes | traffic / algorithmic | "
               "algorithmic GB/s |")
    out.append("|---|---|---|---|---|---|---|")
    stages = (("worker (compress-only)", "worker", "k_compress_onepass<1, ", 16.125),
              ("server", "server", "k_compress_onepass<2, ", a.W / 8 + 12.125))
    for label, _, frag, bpe in stages:
        key = next((k for k in stats if frag in k), None)
        if key is None:
            continue
        ns = float(stats[key]["AverageNs"])
        rd = counter("FETCH_SIZE", frag) * 1024.0 * f_scale
        wr = counter("WRITE_SIZE", frag) * 1024.0 * w_scale
        alg = bpe * a.n
        out.append(f"| {label} | {stats[key]['Calls']} | {ns:.0f} | {rd:.0f} | {wr:.0f} | {(rd + wr) / alg:.4f} | "
                   f"{alg / ns:.0f} |")
    if sq_dir:
        out.append("")
        out.append(f"Issue counters (median per dispatch).  VALU issue bound: {VALU_LANE_OPS_PER_S / 1e12:.2f} T "
                   f"lane-instructions/s (256 CUs x 4 SIMD16 x one wave64 instruction per 4 clocks x 2.4 GHz), so "
                   f"VALU time = SQ_INSTS_VALU x 64 / that; fp64 and transcendental instructions issue at lower "
                   f"rates, so it is a lower bound.  Waiting and VALU-active shares are of SQ_WAVE_CYCLES.")
        out.append("")
        out.append("| launch | " + " | ".join(SQ_COUNTERS) + " | VALU lane-instr per element | VALU-issue time ns | "
                   "VALU time / kernel time | waiting share | VALU-active share |")
        out.append("|---|" + "---|" * (len(SQ_COUNTERS) + 5))
        for label, tag, frag, _ in stages:
            key = next((k for k in stats if frag in k), None)
            vals = {c: counter(c, frag) for c in SQ_COUNTERS}
            if key is None or vals["SQ_INSTS_VALU"] is None:
                continue
            ns = float(stats[key]["AverageNs"])
            per_elem = vals["SQ_INSTS_VALU"] * 64.0 / a.n
            valu_ns = vals["SQ_INSTS_VALU"] * 64.0 / VALU_LANE_OPS_PER_S * 1e9
            wait = vals["SQ_WAIT_ANY"] / vals["SQ_WAVE_CYCLES"] if vals["SQ_WAVE_CYCLES"] else float("nan")
            act = vals["SQ_ACTIVE_INST_VALU"] / vals["SQ_WAVE_CYCLES"] if vals["SQ_WAVE_CYCLES"] else float("nan")
            out.append(f"| {label} | " + " | ".join(f"{vals[c]:.0f}" for c in SQ_COUNTERS) +
                       f" | {per_elem:.2f} | {valu_ns:.0f} | {valu_ns / ns:.3f} | {wait:.3f} | {act:.3f} |")
            out.append(f"<!-- {tag} valu_lane_instr_per_element={per_elem:.4f} -->")
    return "\n".join(out) + "\n"


def allreduce_valu():
    """{"worker"/"server": VALU lane-instructions per element} from the committed
    all-reduce summary, if the library sources still match."""
    try:
        text = open(ALLREDUCE_SUMMARY).read()
    except OSError:
        return {}
    if f"Library source digest: {source_digest()}" not in text:
        return {}
    res = {}
    for line in text.splitlines():
        if line.startswith("<!-- ") and "valu_lane_instr_per_element=" in line:
            label, kv = line[5:-4].split(" ", 1)
            res[label] = float(kv.split("=")[1])
    return res


def _short(name):
    return name.split("(")[0].replace("void ", "").strip()


def summarize_profile(kt_dir, fetch_dir, write_dir):
    """Summary text from rocprofv3 output (kernel trace + stats, FETCH_SIZE, WRITE_SIZE runs)."""
    import numpy as np
    stats = _rows(kt_dir, "kernel_stats.csv")
    out = ["# k_compress_onepass on the BERT-Large-shaped vector (335,143,938 fp32 params)", ""]
    out.append("Commands (from the repository root, on one MI355X):")
    out.append("```")
    for d, extra in ((kt_dir, "--kernel-trace --stats"), (fetch_dir, "--pmc FETCH_SIZE"), (write_dir, "--pmc WRITE_SIZE")):
        out.append(f"rocprofv3 {extra} --output-format csv -d {d} -o bench -- python3 bench.py --profile")
    out.append(f"python bench.py --summarize-profile {kt_dir} {fetch_dir} {write_dir}")
    out.append("```")
    out.append(f"Library source digest: {source_digest()}")
    out.append("")
    out.append("## Kernel time (rocprofv3 --kernel-trace --stats)")
    out.append("")
    out.append("| kernel | calls | average ns | min ns | max ns |")
    out.append("|---|---|---|---|---|")
    for r in stats:
        if "onebit" in r["Name"] or "neg_kernel" in r["Name"]:
            out.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
    res = {}
    for key, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _rows(d, "counter_collection.csv")
        per = {}
        for r in rows:
            if r.get("Counter_Name") != key:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        res[key] = per
    def pick(per, pred, how=np.median):
        vals = [v for k, vs in per.items() if pred(k) for v in vs]
        return float(how(vals)) if vals else None
    onepass = lambda k: "k_compress_onepass" in k  # noqa: E731
    copy = lambda k: "neg_kernel" in k  # noqa: E731
    f_one, w_one = pick(res["FETCH_SIZE"], onepass), pick(res["WRITE_SIZE"], onepass)
    # the calibration copy is the largest copy dispatch of the run
    f_cp, w_cp = pick(res["FETCH_SIZE"], copy, np.max), pick(res["WRITE_SIZE"], copy, np.max)
    cal_bytes = CALIBRATION_FLOATS * 4
    f_scale = cal_bytes / (f_cp * 1024.0) if f_cp else None
    w_scale = cal_bytes / (w_cp * 1024.0) if w_cp else None
    out.append("")
    out.append("## HBM traffic per launch (rocprofv3 --pmc, KiB per dispatch, median over dispatches)")
    out.append("")
    out.append(f"- calibration copy of {cal_bytes} B: FETCH_SIZE {f_cp} KiB, WRITE_SIZE {w_cp} KiB "
               f"-> scale {f_scale:.4f} (fetch), {w_scale:.4f} (write) bytes per counted byte")
    out.append(f"- k_compress_onepass: FETCH_SIZE {f_one} KiB, WRITE_SIZE {w_one} KiB")
    t_read = f_one * 1024.0 * f_scale
    t_write = w_one * 1024.0 * w_scale
    out.append(f"- traffic_read_bytes: {t_read:.0f}")
    out.append(f"- traffic_write_bytes: {t_write:.0f}")
    out.append(f"- traffic_bytes_per_launch: {t_read + t_write:.0f}")
    return "\n".join(out) + "\n"


def profile_traffic():
    """Traffic per launch of the one-pass kernel from the committed summary, if the sources still match."""
    try:
        text = open(PROFILE_SUMMARY).read()
    except OSError:
        return None
    if f"Library source digest: {source_digest()}" not in text:
        return None
    for line in text.splitlines():
        if line.startswith("- traffic_bytes_per_launch:"):
            return float(line.split(":")[1])
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="bert_large", choices=["bert_large", "gpt2_xl"])
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("KT_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--profile-quantizers", action="store_true")
    ap.add_argument("--profile-allreduce", action="store_true")
    ap.add_argument("--summarize-allreduce", nargs="+", metavar="DIR",
                    help="KT_DIR FETCH_DIR WRITE_DIR [SQ_DIR]")
    ap.add_argument("--summarize-quantizers", nargs=2, metavar=("KT_DIR", "PMC_DIR"))
    ap.add_argument("--summarize-kernels", nargs=2, metavar=("KT_DIR", "COMMAND"))
    ap.add_argument("--ceilings", action="store_true")
    ap.add_argument("--placement", action="store_true")
    ap.add_argument("--ceilings-elems", type=int, default=268_435_456,
                    help="fp32 elements per stream for --ceilings (a multiple of 4)")
    args = ap.parse_args()
    if args.ceilings:
        sys.stdout.write(ceilings(args.ceilings_elems))
        return
    if args.placement:
        sys.stdout.write(placement())
        return
    if args.summarize_profile:
        sys.stdout.write(summarize_profile(*args.summarize_profile))
        return
    if args.summarize_kernels:
        sys.stdout.write(summarize_kernels(*args.summarize_kernels))
        return
    if args.summarize_quantizers:
        sys.stdout.write(summarize_quantizers(*args.summarize_quantizers))
        return
    if args.summarize_allreduce:
        sys.stdout.write(summarize_allreduce(*args.summarize_allreduce))
        return
    if args.profile_quantizers:
        profile_quantizers()
        return
    if args.profile_allreduce:
        profile_allreduce(max(1, min(args.steps, 10)))
        return
    if args.profile:
        profile_mode(max(1, min(args.steps, 20)))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the library "
              f"has no multi-GPU path: the compressed all-reduce is simulated inside one GPU's memory)", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)

    import torch
    ensure_built()
    from error_compensated_bit_amd import workloads as W
    dev = "cuda:0"
    torch.cuda.set_device(0)

    wl = W.bert_like() if args.workload == "bert_large" else W.gpt2_like()
    bpe = B_COMPRESS_F32
    log(f"[bench] workload {wl.name}: n={wl.n} chunks={wl.n_chunks}")
    head = bench_compress(wl, args.steps, args.warmup, dev, bpe)
    log(f"[bench] {head['params_per_s'] / 1e9:.1f} G params/s, {head['gbps']:.0f} GB/s algorithmic; "
        f"kernels {head['kernels']}")
    torch.cuda.empty_cache()

    ceiling = stream_ceiling(dev)
    log(f"[bench] streaming ceiling on this device: {ceiling}")
    torch.cuda.empty_cache()

    rows = {}
    if not args.headline_only:
        rows = secondary_rows(dev, args)

    base = None if args.no_cpu_baseline else cpu_baseline(wl, dev)
    if rows and not args.no_cpu_baseline:
        with pinned_to_one_core():
            cpu_row_baselines(rows)
        log(f"[bench] cpu oracle per row: {[(k, round(r['cpu_oracle']['value'], 3)) for k, r in rows.items() if 'cpu_oracle' in r]}")
    if base:
        log(f"[bench] cpu oracle {base['value'] / 1e6:.1f} M params/s on {base['sample']}")

    line = headline_line(wl, bpe, head, base, ceiling, rows, args.steps, args.warmup)
    print(json.dumps(line), flush=True)


def headline_line(wl, bpe, head, base, ceiling, rows, steps, warmup):
    """The one JSON line: the headline measurement (head, from bench_compress), the CPU
    baseline (base, or None), the live streaming ceiling and the other rows."""
    k_ms = head.get("onepass_ms")
    achieved = head.get("onepass_gbps")
    line = {
        "metric": "params/sec and HBM GB/s (% of peak) for fused 1-bit compress+update",
        "value": head["params_per_s"],
        "unit": "params/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": head["seconds_per_call"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "hbm_gbps": head["gbps"],
        "hbm_frac": head["gbps"] / PEAK_HBM_GBPS,
        "config": {"workload": f"{wl.name} flat vector: {wl.n} fp32 params, {wl.n_chunks} chunks "
                               f"(one per tensor), {int((wl.tensor_keep == 0).sum()) if wl.tensor_keep is not None else 0}"
                               f" masked tensors, one compressed step per call",
                   "params": wl.n, "chunks": wl.n_chunks, "grad_dtype": "bf16" if wl.grad_bf16 else "f32",
                   "bytes_per_param": bpe, "plan": head["plan"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": (achieved / PEAK_HBM_GBPS) if achieved else None, "traffic": profile_traffic(),
                     "kernel": "k_compress_onepass (update mode): the dominant kernel, over the "
                               f"{head['onepass_elements']} elements of the one-pass chunks; the whole step, "
                               "two-pass chunk and launch gaps included, is step_frac",
                     "bytes_per_launch": bpe * head["onepass_elements"], "mean_launch_ms": k_ms,
                     "timing": "mean of HIP events recorded around each one-pass launch on its launch stream "
                               "inside the timed steps, the only events there",
                     "step_frac": head["gbps"] / PEAK_HBM_GBPS},
        "cpu_baseline": ({k: base[k] for k in ("value", "unit", "cores", "kind", "sample", "cpu_model", "host_cpus",
                                               "cpus_allowed", "pinned_core")} if base else None),
        "ceiling": dict(ceiling, kernel_frac_of_ceiling=(achieved / ceiling["gbps_5r3w"]) if achieved else None),
        "rows": rows,
    }
    return line


def stream_ceiling(dev, n=335_544_320):
    """Best rate of a plain streaming kernel with the compression kernel's mix (5 fp32
    reads + 3 writes per element) over a few grid sizes, measured now on this device:
    what the HBM delivers for that mix, next to its 8 TB/s peak."""
    import torch
    from error_compensated_bit_amd import onebit as ob
    bufs = [torch.zeros(n, device=dev) for _ in range(8)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = {}
    for name, ins, outs, bpe in (("5r3w", bufs[:5], bufs[5:], 32.0),):
        for block, mults in ((256, (1, 2, 3, 6, 16, 32)), (1024, (1, 2, 4, 6, 8))):
            for mult in mults:
                keep = ob.onebit_stream_probe(ins, outs, cus * mult, block, 1)    # warm
                times = []
                for _ in range(4):
                    ev0.record()
                    keep = ob.onebit_stream_probe(ins, outs, cus * mult, block, 1)
                    ev1.record()
                    ev1.synchronize()
                    times.append(ev0.elapsed_time(ev1))
                del keep
                gbps = bpe * n / (min(times) * 1e-3) / 1e9
                if gbps > best.get(name, (0.0, 0, 0))[0]:
                    best[name] = (gbps, cus * mult, block)
    del bufs
    return {"gbps_5r3w": best["5r3w"][0], "grid_5r3w": best["5r3w"][1], "block_5r3w": best["5r3w"][2],
            "elements": n, "kernel": "onebit_stream_probe"}


CEILING_MIXES = ((1, 0), (0, 1), (1, 1), (2, 1), (3, 1), (1, 2), (2, 2), (4, 2), (5, 3))


def ceilings(n=268_435_456):
    """Streaming ceilings of this device: the plain probe kernel for each read/write
    mix, with the streaming (nontemporal) and the default cache policy, over
    256-thread workgroups (1-32 per CU) and 1024-thread workgroups (1-8 per CU),
    and with its loads staged in LDS by the load unit (256-thread workgroups);
    the best rate of each, and the best with 256-thread workgroups (the compression
    kernels' shape).  Returns the markdown summary kept under profiles/."""
    import torch
    from error_compensated_bit_amd import onebit as ob
    ensure_built()
    dev = "cuda:0"
    bufs = [torch.zeros(n, device=dev) for _ in range(8)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    shapes = [(256, m) for m in (1, 2, 3, 4, 6, 8, 16, 32)] + [(1024, m) for m in (1, 2, 4, 6, 8)]
    out = [f"# Streaming ceilings by read/write mix and cache policy ({n} fp32 elements per stream)", ""]
    out.append("Command (from the repository root, on one MI355X):")
    out.append("```")
    out.append("python bench.py --ceilings" + ("" if n == 268_435_456 else f" --ceilings-elems {n}"))
    out.append("```")
    out.append(f"Device: {torch.cuda.get_device_name(0)}, {cus} CUs.  Kernel: onebit_stream_probe (four 16-byte "
               f"vectors per thread and stream per iteration, grid-stride; with loads staged in LDS, each wave "
               f"double-buffers four 1 KiB global-to-LDS loads per input stream and reads them back).  Bytes "
               f"counted: (reads + writes) x 4 x n per launch; time: best of 4 launches between HIP events on the "
               f"launch stream, after one warm launch.  Peak: {PEAK_HBM_GBPS:.0f} GB/s.")
    out.append("")
    out.append("| reads + writes | cache policy | best GB/s | fraction of 8 TB/s | best shape (threads x WG per CU) | "
               "best GB/s with 256-thread WGs |")
    out.append("|---|---|---|---|---|---|")
    for reads, writes in CEILING_MIXES:
        ins, outs = bufs[:reads], bufs[reads:reads + writes]
        for policy in (1, 0, 2):
            if policy == 2 and reads == 0:
                continue
            best, best256 = (0.0, None), 0.0
            for block, mult in shapes:
                if policy == 2 and block != 256:
                    continue
                keep = ob.onebit_stream_probe(ins, outs, cus * mult, block, policy)
                times = []
                for _ in range(4):
                    ev0.record()
                    keep = ob.onebit_stream_probe(ins, outs, cus * mult, block, policy)
                    ev1.record()
                    ev1.synchronize()
                    times.append(ev0.elapsed_time(ev1))
                del keep
                gbps = (reads + writes) * 4.0 * n / (min(times) * 1e-3) / 1e9
                if gbps > best[0]:
                    best = (gbps, f"{block} x {mult}")
                if block == 256:
                    best256 = max(best256, gbps)
            pol = ("default", "nontemporal", "nontemporal, loads staged in LDS")[policy]
            out.append(f"| {reads} + {writes} | {pol} | {best[0]:.0f} | {best[0] / PEAK_HBM_GBPS:.3f} | {best[1]} | "
                       f"{best256:.0f} |")
            log(f"[ceilings] {reads}+{writes} {pol}: {best[0]:.0f} GB/s ({best[1]}), 256-thread {best256:.0f}")
    del bufs
    return "\n".join(out) + "\n"


def placement():
    """LoCo quantize (4-bit, buckets of 1024, the QSGD workload's 1.3e9-element bf16
    gradient) and the plain streaming probe with two inputs, the second written in
    place (as LoCo's error average is), by the placement of the second buffer: its
    own allocation, or in one allocation at several gaps after the first.  Returns
    the markdown summary kept under profiles/."""
    import torch
    from error_compensated_bit_amd import onebit as ob
    from error_compensated_bit_amd import workloads as W
    ensure_built()
    dev = "cuda:0"
    qg = W.QsgdWorkload()
    n = qg.n
    nb = (n + qg.bucket - 1) // qg.bucket
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best_ms(call, reps=4):
        call()
        ts = []
        for _ in range(reps):
            ev0.record()
            call()
            ev1.record()
            ev1.synchronize()
            ts.append(ev0.elapsed_time(ev1))
        return min(ts)

    gaps_kib = [0, 4, 64, 1024, 2048, 65536]
    out = [f"# Buffer placement: LoCo quantize and an in-place 2-read/1-write stream ({n} elements)", ""]
    out.append("Command (from the repository root, on one MI355X):")
    out.append("```")
    out.append("python bench.py --placement")
    out.append("```")
    out.append("LoCo: 4-bit codes, buckets of 1024, bf16 gradient (N(0, 1) x 10^U(-4, -2) per 2^20 block), fp32 error "
               "average updated in place, beta 0.9; best of 4 calls between HIP events.  Stream: onebit_stream_probe "
               f"over {n // 4} fp32 elements per stream, inputs a and b, output b (in place), nontemporal, best of "
               "grids 4 and 6 per CU.")
    out.append("")
    out.append("| second buffer | LoCo ms | LoCo G elem/s | stream GB/s |")
    out.append("|---|---|---|---|")
    codes = torch.zeros((n + 1) // 2, dtype=torch.uint8, device=dev)
    norms = torch.zeros(nb, device=dev)
    g = W.qsgd_gradient(qg, 0, device=dev)
    ns = n // 4
    pool = torch.zeros(2 * n + max(gaps_kib) * 1024 + 4 * n + 4096, dtype=torch.uint8, device=dev)

    def stream_gbps(a, b):
        ms = min(best_ms(lambda m=m: ob.onebit_stream_probe([a, b], [b], cus * m, 256, 1), 3) for m in (4, 6))
        return 12.0 * ns / (ms * 1e-3) / 1e9

    e = torch.zeros(n, device=dev)
    t = best_ms(lambda: ob.loco_quantize(g, e, qg.bucket, 4, 0.9, 7, codes, norms))
    a_sep, b_sep = e[:ns], torch.zeros(ns, device=dev)
    out.append(f"| own allocation | {t:.3f} | {n / t / 1e6:.0f} | {stream_gbps(a_sep, b_sep):.0f} |")
    log(f"[placement] separate: {t:.3f} ms")
    del e, a_sep, b_sep
    gv = pool[:2 * n].view(torch.bfloat16)
    gv.copy_(g)
    del g
    torch.cuda.empty_cache()
    spool = torch.zeros(8 * ns + max(gaps_kib) * 1024 + 4096, dtype=torch.uint8, device=dev)   # the stream's own
    for gap in gaps_kib:
        start = (2 * n + gap * 1024 + 255) // 256 * 256
        ev_ = pool[start:start + 4 * n].view(torch.float32)
        t = best_ms(lambda: ob.loco_quantize(gv, ev_, qg.bucket, 4, 0.9, 7, codes, norms))
        a = spool[:4 * ns].view(torch.float32)
        sb = (4 * ns + gap * 1024 + 255) // 256 * 256
        b = spool[sb:sb + 4 * ns].view(torch.float32)
        out.append(f"| same allocation, {gap} KiB after the first | {t:.3f} | {n / t / 1e6:.0f} | {stream_gbps(a, b):.0f} |")
        log(f"[placement] gap {gap} KiB: {t:.3f} ms")
    del pool, spool
    return "\n".join(out) + "\n"


def roof(gbps, elems_per_s=None, label=None, valu=None, rng=None):
    """Roofline of a row: HBM fraction of 8 TB/s, and for the quantizers the fraction of
    the VALU issue-rate bound (from the committed instruction counts); bound = the
    larger fraction.  rng: the element rate that drawing the quantizer's random
    numbers alone reaches (the Philox probe), reported beside it."""
    r = {"hbm_frac": gbps / PEAK_HBM_GBPS}
    per = (valu or {}).get(label)
    if per and elems_per_s:
        r["alu_peak_elems_per_s"] = VALU_LANE_OPS_PER_S / per
        r["alu_frac"] = elems_per_s / r["alu_peak_elems_per_s"]
    if rng and elems_per_s:
        r["rng_only_elems_per_s"] = rng
        r["rng_frac"] = elems_per_s / rng
    r["bound"] = "alu" if r.get("alu_frac", 0.0) > r["hbm_frac"] else "hbm"
    return r


def philox_ceiling(dev, n_elems):
    """Elements per second that drawing Philox4x32-10 numbers alone allows (one block
    of four words per four elements, as the quantizers draw them): the Philox probe
    over n_elems / 4 blocks, best grid, best of 3 launches each."""
    import torch
    from error_compensated_bit_amd import onebit as ob
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_blocks = (n_elems + 3) // 4
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = (0.0, None)
    for block, mults in ((256, (2, 4, 8, 16, 32)), (1024, (1, 2, 4, 8))):
        for mult in mults:
            out = torch.empty(cus * mult * block, dtype=torch.int32, device=dev)
            ob.onebit_philox_probe(0, n_blocks, out, cus * mult, block)
            times = []
            for _ in range(3):
                ev0.record()
                ob.onebit_philox_probe(0, n_blocks, out, cus * mult, block)
                ev1.record()
                ev1.synchronize()
                times.append(ev0.elapsed_time(ev1))
            rate = n_elems / (min(times) * 1e-3)
            if rate > best[0]:
                best = (rate, f"{block} x {mult}")
    return {"elems_per_s": best[0], "blocks_per_s": best[0] / 4.0, "shape": best[1], "elements": n_elems,
            "kernel": "onebit_philox_probe"}


def secondary_rows(dev, args):
    import numpy as np
    import torch
    from error_compensated_bit_amd import onebit as ob
    from error_compensated_bit_amd import workloads as W
    rows = {}
    steps = max(3, args.steps // 3)
    valu = valu_per_element()

    # warmup Adam step on the BERT-Large-sized vector
    n = 335_143_938
    x = torch.zeros(n, device=dev)
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    g = torch.randn(n, device=dev) * 1e-3

    def warm():
        ob.onebit_adam_warmup_step(x, m, v, g, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                                   bias_correction=False, step=1)
    t, kt = timed(warm, steps, 2)
    km = kt.mean_ms("warmup")
    rows["warmup_adam_bert_large"] = dict(params_per_s=n / t, gbps=B_WARMUP * n / t / 1e9,
                                          kernel_gbps=B_WARMUP * n / (km * 1e-3) / 1e9,
                                          roofline=roof(B_WARMUP * n / (km * 1e-3) / 1e9))
    del x, m, v, g
    torch.cuda.empty_cache()
    log(f"[bench] warmup {rows['warmup_adam_bert_large']}")

    # QSDP on 1.3e9 bf16 weights
    q = W.QsdpWorkload()
    rng = philox_ceiling(dev, q.n)
    rows["philox4x32_10_only"] = rng
    log(f"[bench] philox only {rng}")
    xq = W.qsdp_weights(q, device=dev)
    nb = (q.n + q.bucket - 1) // q.bucket
    bmin = torch.zeros(nb, device=dev)
    bmax = torch.zeros(nb, device=dev)
    for bits, bpe in ((4, B_QSDP4), (8, B_QSDP8)):
        codes = torch.zeros(q.n if bits == 8 else (q.n + 1) // 2, dtype=torch.uint8, device=dev)
        out = torch.zeros(q.n, dtype=torch.bfloat16, device=dev)
        tq, ktq = timed(lambda: ob.qsdp_quantize(xq, q.bucket, bits, 0, codes, bmin, bmax), steps, 1)
        td, ktd = timed(lambda: ob.qsdp_dequantize(codes, bmin, bmax, q.n, q.bucket, bits, out), steps, 1)
        rows[f"qsdp{bits}_quantize"] = dict(elems_per_s=q.n / tq, gbps=bpe * q.n / tq / 1e9)
        rows[f"qsdp{bits}_quantize"]["roofline"] = roof(bpe * q.n / tq / 1e9, q.n / tq, f"qsdp{bits}_quantize", valu,
                                                         rng["elems_per_s"])
        rows[f"qsdp{bits}_dequantize"] = dict(elems_per_s=q.n / td, gbps=bpe * q.n / td / 1e9)
        rows[f"qsdp{bits}_dequantize"]["roofline"] = roof(bpe * q.n / td / 1e9)
        del codes, out
    # one seed of the 64-seed error statistic (4-bit): quantize, dequantize to fp32,
    # then the statistic (sums of y - x and (y - x)^2, ysum += y); the mean absolute
    # error of the seed average runs once after the 64 seeds
    codes = torch.zeros((q.n + 1) // 2, dtype=torch.uint8, device=dev)
    y = torch.zeros(q.n, device=dev)
    ysum = torch.zeros(q.n, dtype=torch.float64, device=dev)
    sums = torch.zeros(2, dtype=torch.float64, device=dev)
    part = torch.zeros(2 * ob.QSDP_STATS_PARTIALS, dtype=torch.float64, device=dev)
    mae = torch.zeros(1, dtype=torch.float64, device=dev)
    seed = [0]

    def one_seed():
        ob.qsdp_quantize(xq, q.bucket, 4, seed[0], codes, bmin, bmax)
        ob.qsdp_dequantize(codes, bmin, bmax, q.n, q.bucket, 4, None, y)
        ob.qsdp_error_stats(xq, y, ysum, sums, part)
        seed[0] += 1
    ts, kts = timed(one_seed, steps, 1)
    tm, _ = timed(lambda: ob.qsdp_mean_abs_error(xq, ysum, q.seeds, mae, part), steps, 1)
    st_ms = kts.mean_ms("finalize")
    rows["qsdp4_seed_statistic"] = dict(
        ms_per_seed=ts * 1e3, elems_per_s=q.n / ts, ms_64_seeds=(q.seeds * ts + tm) * 1e3,
        statistic_kernel_gbps=B_QSDP_STAT * q.n / (st_ms * 1e-3) / 1e9,
        mean_abs_error_gbps=B_QSDP_MAE * q.n / tm / 1e9,
        roofline=roof(B_QSDP_STAT * q.n / (st_ms * 1e-3) / 1e9))
    del codes, y, ysum
    del xq, bmin, bmax
    torch.cuda.empty_cache()
    log(f"[bench] qsdp {[(k, v) for k, v in rows.items() if 'qsdp' in k]}")

    # QSGD on the same model's bf16 gradients: one worker's quantization of its whole
    # gradient, then the shard owner's decode-and-average of 8 workers' streams
    qg = W.QsgdWorkload()
    gq = W.qsgd_gradient(qg, 0, device=dev)
    nbq = (qg.n + qg.bucket - 1) // qg.bucket
    norms = torch.zeros((qg.W, nbq), device=dev)
    for bits in (4, 8):
        cb = (qg.n + 1) // 2 if bits == 4 else qg.n
        stride = (cb + 15) // 16 * 16
        codes = torch.zeros((qg.W, stride), dtype=torch.uint8, device=dev)
        for w in range(qg.W):
            ob.qsgd_quantize(gq, qg.bucket, bits, 100 + w, codes[w], norms[w])
        out = torch.zeros(qg.shard, device=dev)
        tq, _ = timed(lambda: ob.qsgd_quantize(gq, qg.bucket, bits, 7, codes[0], norms[0]), steps, 1)
        tr, _ = timed(lambda: ob.qsgd_reduce(codes, norms, qg.shard, qg.bucket, bits, out_f32=out), steps, 1)
        bq = 2.0 + bits / 8.0 + 4.0 / qg.bucket
        br = qg.W * (bits / 8.0 + 4.0 / qg.bucket) + 4.0
        rows[f"qsgd{bits}_quantize"] = dict(elems_per_s=qg.n / tq, gbps=bq * qg.n / tq / 1e9,
                                            roofline=roof(bq * qg.n / tq / 1e9, qg.n / tq, f"qsgd{bits}_quantize", valu,
                                                          rng["elems_per_s"]))
        rows[f"qsgd{bits}_reduce_{qg.W}x{qg.shard}"] = dict(elems_per_s=qg.shard / tr, gbps=br * qg.shard / tr / 1e9,
                                                            roofline=roof(br * qg.shard / tr / 1e9))
        if bits == 4:
            err = torch.zeros(qg.n, device=dev)
            tl, _ = timed(lambda: ob.loco_quantize(gq, err, qg.bucket, bits, 0.9, 7, codes[0], norms[0]), steps, 1)
            rows["loco4_quantize"] = dict(elems_per_s=qg.n / tl, gbps=(bq + 8.0) * qg.n / tl / 1e9,
                                          roofline=roof((bq + 8.0) * qg.n / tl / 1e9, qg.n / tl, "loco4_quantize", valu,
                                                        rng["elems_per_s"]))
            del err
        del codes, out
    del gq, norms
    torch.cuda.empty_cache()
    log(f"[bench] qsgd {[(k, v) for k, v in rows.items() if 'qsgd' in k]}")

    # simulated compressed all-reduce: 16 workers x 64M fp32, 16 chunks of 4M
    a = W.AllreduceWorkload()
    ar_valu = allreduce_valu()
    plan = ob.onebit_plan_create(a.chunk_off)
    words, nch = ob.onebit_plan_words(plan), ob.onebit_plan_chunks(plan)
    m = torch.zeros(a.n, device=dev)
    e = torch.zeros((a.W, a.n), device=dev)
    es = torch.zeros(a.n, device=dev)
    grads = torch.randn((a.W, a.n), device=dev) * a.grad_std
    wbits = torch.zeros((a.W, words), dtype=torch.int32, device=dev)
    wsc = torch.zeros((a.W, nch), device=dev)
    sbits = torch.zeros(words, dtype=torch.int32, device=dev)
    ssc = torch.zeros(nch, device=dev)
    wsp = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=dev)

    def allreduce_step():
        for w in range(a.W):
            ob.onebit_compress_update(plan, grads[w], m, e[w], None, None, None, wbits[w], wsc[w], lr=0.0,
                                      beta1=0.9, eps=1e-8, weight_decay=0.0, workspace=wsp)
        ob.onebit_server_reduce(plan, wbits, wsc, es, sbits, ssc, m, wsp)
    t, kt = timed(allreduce_step, steps, 1)
    w_ms = kt.mean_ms("compress_onepass")
    s_ms = kt.mean_ms("server_onepass")
    # the same 17 launches captured once in a HIP graph and replayed
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        allreduce_step()
    t_graph, _ = timed(graph.replay, steps, 1)
    del graph
    step_bytes = (B_WORKER * a.W + 14.125) * a.n
    rows["allreduce_16x64M"] = dict(ms_per_step=t * 1e3, gbps=step_bytes / t / 1e9,
                                    worker_kernel_gbps=B_WORKER * a.n / (w_ms * 1e-3) / 1e9,
                                    server_kernel_gbps=14.125 * a.n / (s_ms * 1e-3) / 1e9,
                                    server_kernel_ms=s_ms, worker_kernel_ms=w_ms,
                                    ms_per_step_graph_replay=t_graph * 1e3,
                                    worker_roofline=roof(B_WORKER * a.n / (w_ms * 1e-3) / 1e9, a.n / (w_ms * 1e-3),
                                                         "worker", ar_valu),
                                    server_roofline=roof(14.125 * a.n / (s_ms * 1e-3) / 1e9, a.n / (s_ms * 1e-3),
                                                         "server", ar_valu))
    # the same exchange as a full step: fp16 gradients, the server's result masked
    # per element into the momentum, frozen-v update of x
    g16 = grads.to(torch.float16)
    del grads
    v = torch.rand(a.n, device=dev) * 1e-6 + 1e-7
    x = torch.randn(a.n, device=dev) * 0.02
    mask = (torch.rand(a.n, device=dev) < 0.98).to(torch.uint8)

    def full_step():
        for w in range(a.W):
            ob.onebit_compress_update(plan, g16[w], m, e[w], None, None, None, wbits[w], wsc[w], lr=0.0,
                                      beta1=0.9, eps=1e-8, weight_decay=0.0, workspace=wsp)
        ob.onebit_server_reduce(plan, wbits, wsc, es, sbits, ssc, m, wsp)
        ob.onebit_momentum_update(m, mask, v, x, None, lr=1e-3, eps=1e-8, weight_decay=0.01)
    t, kt = timed(full_step, steps, 1)
    f_ms = kt.mean_ms("momentum_update")
    step_bytes = (B_WORKER_F16 * a.W + 14.125 + B_FINISH_MASK) * a.n
    rows["full_step_16x64M_f16_mask"] = dict(ms_per_step=t * 1e3, gbps=step_bytes / t / 1e9,
                                             worker_kernel_gbps=B_WORKER_F16 * a.n /
                                             (kt.mean_ms("compress_onepass") * 1e-3) / 1e9,
                                             finish_kernel_gbps=B_FINISH_MASK * a.n / (f_ms * 1e-3) / 1e9,
                                             finish_kernel_ms=f_ms,
                                             finish_roofline=roof(B_FINISH_MASK * a.n / (f_ms * 1e-3) / 1e9))
    # the same full step with the momentum kept as the server's words and scales
    pb = [sbits, torch.zeros_like(sbits)]
    pss = [ssc, torch.zeros_like(ssc)]
    flip = [0]

    def full_step_packed():
        c = flip[0]
        for w in range(a.W):
            ob.onebit_compress_update_packed(plan, g16[w], pb[c], pss[c], e[w], None, None, None, wbits[w], wsc[w],
                                             lr=0.0, beta1=0.9, eps=1e-8, weight_decay=0.0, workspace=wsp,
                                             m_mask=mask)
        ob.onebit_server_reduce(plan, wbits, wsc, es, pb[1 - c], pss[1 - c], None, wsp)
        ob.onebit_momentum_update_packed(plan, pb[1 - c], pss[1 - c], mask, v, x, None, lr=1e-3, eps=1e-8,
                                         weight_decay=0.01)
        flip[0] = 1 - c
    t, kt = timed(full_step_packed, steps, 1)
    assert ob.onebit_workspace_status(wsp) == 0
    step_bytes = ((B_WORKER_F16 - 4.0 + 1.125) * a.W + 10.125 + B_FINISH_PACKED) * a.n
    rows["full_step_16x64M_f16_mask_packed_m"] = dict(ms_per_step=t * 1e3, gbps=step_bytes / t / 1e9,
                                                      finish_kernel_ms=kt.mean_ms("momentum_update"))
    # one GPU's share of the same step on 16 GPUs: its own worker over the whole
    # vector, the server stage over its 4M-element shard with 16 workers' streams of
    # that shard, and the finish over the whole vector (the all-gather between them is
    # not simulated); fp32 momentum, then the packed momentum
    shard = int(a.chunk_off[1])
    plan_s = ob.onebit_plan_create(np.array([0, shard], np.int64))
    ws_s = torch.zeros(ob.onebit_plan_workspace_bytes(plan_s) // 8, dtype=torch.int64, device=dev)
    sw = ob.onebit_plan_words(plan_s)
    wbits_s = wbits[:, :sw].contiguous()
    wsc_s = wsc[:, :1].contiguous()
    es_s = torch.zeros(shard, device=dev)
    sb_s, ss_s, mo_s = torch.zeros(sw, dtype=torch.int32, device=dev), torch.zeros(1, device=dev), \
        torch.zeros(shard, device=dev)

    def gpu_share():
        ob.onebit_compress_update(plan, g16[0], m, e[0], None, None, None, wbits[0], wsc[0], lr=0.0, beta1=0.9,
                                  eps=1e-8, weight_decay=0.0, workspace=wsp)
        ob.onebit_server_reduce(plan_s, wbits_s, wsc_s, es_s, sb_s, ss_s, mo_s, ws_s)
        ob.onebit_momentum_update(m, mask, v, x, None, lr=1e-3, eps=1e-8, weight_decay=0.01)

    def gpu_share_packed():
        c = flip[0]
        ob.onebit_compress_update_packed(plan, g16[0], pb[c], pss[c], e[0], None, None, None, wbits[0], wsc[0],
                                         lr=0.0, beta1=0.9, eps=1e-8, weight_decay=0.0, workspace=wsp, m_mask=mask)
        ob.onebit_server_reduce(plan_s, wbits_s, wsc_s, es_s, sb_s, ss_s, None, ws_s)
        ob.onebit_momentum_update_packed(plan, pb[c], pss[c], mask, v, x, None, lr=1e-3, eps=1e-8,
                                         weight_decay=0.01)
    t1, _ = timed(gpu_share, steps, 1)
    t2, _ = timed(gpu_share_packed, steps, 1)
    rows["gpu_share_of_16_64M_f16_mask"] = dict(ms_per_step=t1 * 1e3, params_per_s=a.n / t1)
    rows["gpu_share_of_16_64M_f16_mask_packed_m"] = dict(ms_per_step=t2 * 1e3, params_per_s=a.n / t2)
    del m, e, es, v, wbits, wsc, sbits, ssc, wsp, plan, pb, pss, plan_s, ws_s, wbits_s, wsc_s, es_s
    torch.cuda.empty_cache()
    # the same full step through the driver (OneBitAdamWorkers: worker and server
    # errors, element mask, packed momentum after its first compressed step); the
    # error word is read once after the timed steps instead of after every step
    from error_compensated_bit_amd.optimizer import OneBitAdamWorkers
    drv = OneBitAdamWorkers(x, a.W, chunk_offsets=a.chunk_off, exp_avg_mask=mask, lr=1e-3, eps=1e-8,
                            weight_decay=0.01, freeze_step=0, packed_momentum=True, check_every=0)
    drv.v.copy_(torch.rand(a.n, device=dev) * 1e-6 + 1e-7)
    gd = drv.gradient_buffer(torch.float16)
    gd.copy_(g16)
    del g16
    t, _ = timed(lambda: drv.step(gd), steps, 2)
    drv.check()
    rows["driver_workers_16x64M_f16_mask_packed_m"] = dict(ms_per_step=t * 1e3, params_per_s=a.n / t)
    del drv, gd, x, mask
    torch.cuda.empty_cache()
    log(f"[bench] allreduce {rows['allreduce_16x64M']} full step {rows['full_step_16x64M_f16_mask']} "
        f"packed {rows['full_step_16x64M_f16_mask_packed_m']} one GPU's share "
        f"{rows['gpu_share_of_16_64M_f16_mask']} packed {rows['gpu_share_of_16_64M_f16_mask_packed_m']}")

    # the headline step with the momentum kept as the previous step's words and scales
    wl = W.bert_like()
    x, m, e, v = W.init_state(wl, device=dev)
    g = W.gradient(wl, 1, device=dev)
    plan = ob.onebit_plan_create(wl.chunk_off, wl.tensor_off, wl.tensor_keep)
    words, nch = ob.onebit_plan_words(plan), ob.onebit_plan_chunks(plan)
    wsp = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=dev)
    pb = [torch.zeros(words, dtype=torch.int32, device=dev) for _ in range(2)]
    ps = [torch.zeros(nch, device=dev) for _ in range(2)]
    hp = dict(lr=wl.hyper["lr"], beta1=wl.hyper["beta1"], eps=wl.hyper["eps"], weight_decay=wl.hyper["weight_decay"])
    ob.onebit_compress_update(plan, g, m, e, v, x, None, pb[0], ps[0], workspace=wsp, **hp)
    del m
    flip = [0]

    def packed_step():
        c = flip[0]
        ob.onebit_compress_update_packed(plan, g, pb[c], ps[c], e, v, x, None, pb[1 - c], ps[1 - c], workspace=wsp,
                                         **hp)
        flip[0] = 1 - c
    t, kt = timed(packed_step, steps, 1)
    assert ob.onebit_workspace_status(wsp) == 0
    n1 = onepass_elements(wl, plan)
    k_ms = kt.mean_ms("compress_onepass")
    rows["compress_bert_large_packed_m"] = dict(params_per_s=wl.n / t, gbps=B_COMPRESS_PACKED * wl.n / t / 1e9,
                                                onepass_gbps=B_COMPRESS_PACKED * n1 / (k_ms * 1e-3) / 1e9,
                                                roofline=roof(B_COMPRESS_PACKED * n1 / (k_ms * 1e-3) / 1e9))
    del x, e, v, g, pb, ps, wsp, plan
    torch.cuda.empty_cache()
    log(f"[bench] packed momentum {rows['compress_bert_large_packed_m']}")

    # GPT-2-XL-shaped vector, bf16 gradients, bf16 copy of x
    wl = W.gpt2_like()
    r = bench_compress(wl, steps, 1, dev, B_COMPRESS_BF16_COPY)
    rows["compress_gpt2_xl_bf16"] = {k: r[k] for k in ("params_per_s", "gbps", "onepass_gbps", "plan")
                                     if k in r}
    if r.get("onepass_gbps"):
        rows["compress_gpt2_xl_bf16"]["roofline"] = roof(r["onepass_gbps"])
    torch.cuda.empty_cache()
    log(f"[bench] gpt2 {rows['compress_gpt2_xl_bf16']}")
    return rows


if __name__ == "__main__":
    main()
