#!/usr/bin/env python3
"""Throughput of one tensor-parallel rank's MLP forward + backward on one MI355X.

A step is one pass of the whole path over one batch: tp_mlp_fwd (F1: X A_i
with fused bias + GeLU, F2: H_i B_i) then tp_mlp_bwd (B1: dY B_i^T with fused
gelu' and db1 partials, B5: db1 finish, B2: dB, B3: dA, B4: dXp). Inputs are
seeded synthetic tensors resident in HBM before timing starts.

Prints one JSON line: whole-step TFLOP/s (GEMM flops 12 T h f per step over
wall-clock time between device synchronizations), the fraction of the dense
16-bit MFMA peak, the dominant kernel's roofline (its algorithmic flops over
its average duration from HIP events recorded on the launch stream around it
in the timed steps), and the float64 CPU oracle timed on a bounded token
sample of the same workload. The per-kernel breakdown (kernel_ms and the
step medians) comes from as many untimed steps with every step boundary
recorded: an event record between two kernels idles the stream for a few
microseconds, so the timed steps record only the two they need.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s + % MFMA peak, TP-shard MLP fwd+bwd (h=2560..10240), 1 MI355X"
# Dense MFMA peaks of MI355X in TFLOP/s: 256 CUs x 2.4 GHz x 4096 flop/clk/CU
# for fp16/bf16; the fp32 figure is the vector (FMA) peak the fp32 path uses.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
FWD_STEPS = ["TA", "F1", "TB", "F2"]                               # what the 5 forward events bracket
BWD_STEPS = ["B1", "B5", "TH", "TdY", "B2", "TX", "TdZ", "B3", "B4"]  # ... and the 10 backward events
GEMM_STEPS = ["F1", "F2", "B1", "B2", "B3", "B4"]
PROFILE_TAG = {"gpt_h10240": "h10240_bf16"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload_name(cfg):
    return (f"{cfg.name}: one TP={cfg.tp} shard of an MLP with hidden {cfg.hidden}, FFN {cfg.ffn}; "
            f"tokens {cfg.tokens} (micro-batch {cfg.micro_batch} x seq {cfg.seq_len}), shard width {cfg.ffn_shard}")


# The attention shard's own sources: not part of the MLP kernels whose
# counters the profile summary holds.
ATTN_ONLY_SOURCES = {"tp_attn.hip", "tp_attn_flash.hip", "flash_attn.hpp", "attn_common.hpp"}


def source_hash():
    """sha256 over the HIP sources the MLP kernels are built from (csrc/*
    except the attention-only file), in name order."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "megatron_tensor_transformer_04_amd", "csrc", "*"))):
        if os.path.basename(p) in ATTN_ONLY_SOURCES:
            continue
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(cfg_name, step):
    """HBM bytes per launch of `step` (read + write) from the rocprofv3 counter
    summary of this workload under profiles/, or None when there is none or
    the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"gemm_dma_{PROFILE_TAG.get(cfg_name, cfg_name)}.md")
    if not os.path.exists(path):
        return None
    want, vals = None, {}
    with open(path) as f:
        for line in f:
            if line.startswith("traffic-source-sha256:"):
                want = line.split(":", 1)[1].strip()
            elif line.startswith("traffic "):
                parts = line.split()
                kv = dict(x.split("=") for x in parts[2:])
                vals[parts[1]] = int(kv["read_bytes"]) + int(kv["write_bytes"])
    if want != source_hash() or step not in vals:
        return None
    return vals[step]


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(inp, cfg, target_s):
    """The float64 oracle (as it stands) on the first Ts tokens of the same
    workload, Ts chosen so that the timed run takes roughly target_s."""
    import oracle
    h, f = inp.X.shape[1], inp.A.shape[1]

    def run(ts):
        # the backward reuses the forward's Z (as the GPU path does), so the
        # timed work is exactly the 12 T h f of one step
        t0 = time.perf_counter()
        fw = oracle.shard_forward(inp.X[:ts], inp.A, inp.b1, inp.B)
        oracle.shard_backward(inp.X[:ts], inp.A, inp.b1, inp.B, inp.dY[:ts], Z_i=fw["Z"])
        return time.perf_counter() - t0

    probe = min(64, inp.X.shape[0])
    dt = run(probe)
    ts = int(probe * target_s / max(dt, 1e-3)) // 8 * 8
    ts = max(probe, min(ts, inp.X.shape[0]))
    log(f"cpu baseline: oracle on {ts} tokens (probe {probe} tokens took {dt:.2f} s)")
    dt = run(ts)
    flops = 12.0 * ts * h * f
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"float64 NumPy oracle, forward+backward of the same shard on the first {ts} of {cfg.tokens} "
                  f"tokens (same weights), {dt:.1f} s",
    }


def reduce_partials_rate(tpmlp, Yp, cfg, dev, reps=10):
    """HBM rate of tp_mlp_reduce_partials on the TP group's partials of this
    workload: tp partials [T, h] (+ b2) -> Y [T, h], timed with HIP events
    on the launch stream. Not part of a step (the sum over ranks is the
    caller's); reported beside it."""
    import torch
    T, h = Yp.shape
    parts = [Yp] + [torch.empty_like(Yp).copy_(Yp) for _ in range(cfg.tp - 1)]
    b2 = torch.zeros((h,), dtype=Yp.dtype, device=dev)
    out = torch.empty_like(Yp)
    for _ in range(2):
        tpmlp.tp_mlp_reduce_partials(parts, b2, out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        tpmlp.tp_mlp_reduce_partials(parts, b2, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = (cfg.tp + 1) * T * h * Yp.element_size() + h * Yp.element_size()
    del parts, out
    return {"parts": cfg.tp, "ms": round(ms, 4), "bytes": nbytes, "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "peak": 8000.0, "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / 1e9 / 8000.0, 4)}


OTHER_CONFIGS = ("gpt2_small", "gpt_2p4b", "gpt_7b")


def config_rate(tpmlp, name, dev, steps=20, warmup_s=0.1):
    """Whole-step rate of another MLP workload (default launch configuration:
    staged workspaces, H and dZ kept), timed with HIP events on the launch
    stream; reported beside the main workload, whose line this is. Run
    before the main workload, after untimed steps for about warmup_s of GPU
    time (the main workload runs that long, warm-up and breakdown pass,
    before its timed steps), so that neither starts at the clock the other
    leaves the chip at."""
    import torch
    import synth
    from synth.device import device_inputs
    cfg = synth.get_config(name)
    T, h, f = cfg.tokens, cfg.hidden, cfg.ffn_shard
    inp = synth.draw_config(cfg)
    X, A, b1, B, dY = device_inputs(inp)
    td = X.dtype
    e = lambda *s: torch.empty(s, dtype=td, device=dev)
    Z, H, Yp, dZ, dXp, dA, dB, db1 = e(T, f), e(T, f), e(T, h), e(T, f), e(T, h), e(h, f), e(f, h), e(f)
    code = {"f32": tpmlp.TPMLP_F32, "f16": tpmlp.TPMLP_F16, "bf16": tpmlp.TPMLP_BF16}[cfg.dtype]
    nws, nfws = tpmlp.tp_mlp_workspace_bytes(T, h, f, code), tpmlp.tp_mlp_fwd_workspace_bytes(T, h, f, code)
    ws = torch.empty((max(nws, 1),), dtype=torch.uint8, device=dev)
    fws = torch.empty((nfws,), dtype=torch.uint8, device=dev) if nfws else None

    def step():
        tpmlp.tp_mlp_fwd(X, A, b1, B, Z, H, Yp, fws)
        tpmlp.tp_mlp_bwd(dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, ws)

    t0 = time.perf_counter()
    while True:
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= warmup_s:
            break
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # cold caches: a 512 MiB buffer (twice the MALL) is written between steps, each step timed alone
    flush = torch.empty((512 << 20,), dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(5):
        flush.fill_(1)
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        z.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(z))
    del flush
    cold_ms = sorted(cold)[len(cold) // 2]
    flops = 12.0 * T * h * f
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": workload_name(cfg), "dtype": cfg.dtype, "ms_per_step": round(ms, 4),
            "tflops": round(tflops, 2), "pct_of_peak": round(100.0 * tflops / PEAK_TFLOPS[cfg.dtype], 2),
            "cold_ms_per_step": round(cold_ms, 4), "cold_tflops": round(flops / (cold_ms * 1e-3) / 1e12, 2)}


def attention_cpu_baseline(inp, cfg, flops_per_call, target_s=8.0, max_calls=4):
    """The float64 attention oracle (as it stands) on the whole shard (all
    sequences and heads), forward + backward, repeated until about target_s
    of CPU work (at most max_calls calls). flops_per_call counts the work the
    oracle does: its backward recomputes the forward first."""
    import oracle
    b, n = cfg.micro_batch, cfg.heads_shard
    calls, t0 = 0, time.perf_counter()
    while calls < max_calls and (calls == 0 or time.perf_counter() - t0 < target_s):
        oracle.attn_shard_forward(inp.X, inp.Wqkv, inp.bqkv, inp.Wo, b, n, cfg.causal)
        oracle.attn_shard_backward(inp.X, inp.Wqkv, inp.bqkv, inp.Wo, inp.dY, b, n, cfg.causal)
        calls += 1
    dt = time.perf_counter() - t0
    return {"value": calls * flops_per_call / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"float64 NumPy oracle, forward+backward of the whole shard ({b} sequences of {cfg.seq_len} "
                      f"tokens, {n} heads; the backward recomputes the forward, counted), {calls} call(s), "
                      f"{dt:.1f} s"}


def attention_rate(tpmlp, dev, reps=10):
    """Forward + backward of one TP rank's attention share of the 2.4B model
    (8 of 32 heads of width 80, 4 sequences of 2048 tokens, bf16, causal),
    timed with HIP events on the launch stream, through the fused path
    (tp_attn_flash_fwd / tp_attn_flash_bwd: the reported rate) and through
    the materialized one (tp_attn_fwd / tp_attn_bwd, P stored: reported
    beside it). Not part of a step (the MLP block is).
    Algorithmic flops: per pass 2 T h 3q + 2 T q h for the projections and
    2 x 2 Z s^2 d for the scores and P V, halved under the causal mask (the
    products that only meet masked entries are not work); the backward is
    twice the forward (the fused backward's recomputation of the scores is
    not counted)."""
    import torch
    import synth
    from synth.device import to_device
    cfg = synth.get_attn_config("attn_2p4b")
    b, s, h, n, d = cfg.micro_batch, cfg.seq_len, cfg.hidden, cfg.heads_shard, cfg.head_dim
    inp = synth.draw_attn_inputs(b, s, h, n, d, cfg.dtype, seed=cfg.seed, sigma_dy=cfg.sigma_dy)
    X, Wqkv, bqkv, Wo, dY = (to_device(getattr(inp, k), cfg.dtype) for k in ("X", "Wqkv", "bqkv", "Wo", "dY"))
    code = tpmlp.TPMLP_BF16
    u8 = lambda nbytes: torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    T, q, Z = b * s, n * d, b * n
    e = lambda *shape: torch.empty(shape, dtype=X.dtype, device=dev)
    QKV, O, Yp = e(T, 3 * q), e(T, q), e(T, h)
    dQKV, dXp, dWqkv, dbqkv, dWo = e(T, 3 * q), e(T, h), e(h, 3 * q), e(3 * q), e(q, h)
    LSE = torch.empty((Z, s), dtype=torch.float32, device=dev)
    kw = dict(batch=b, heads=n, causal=cfg.causal)

    def measure(fwd, bwd):
        """(forward ms, backward ms, forward + backward ms): the split from
        events around each call, the sum from one event pair around reps
        back-to-back calls (an event record idles the stream for a few
        microseconds, which the split's intervals include)."""
        for _ in range(2):
            fwd()
            bwd()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        torch.cuda.synchronize()
        for r in range(reps):
            ev[r][0].record()
            fwd()
            ev[r][1].record()
            bwd()
            ev[r][2].record()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for r in range(reps):
            fwd()
            bwd()
        g1.record()
        torch.cuda.synchronize()
        return (sum(x[0].elapsed_time(x[1]) for x in ev) / reps, sum(x[1].elapsed_time(x[2]) for x in ev) / reps,
                g0.elapsed_time(g1) / reps)

    ffws = u8(tpmlp.tp_attn_flash_fwd_workspace_bytes(b, s, h, n, d, code, cfg.causal))
    fbws = u8(tpmlp.tp_attn_flash_bwd_workspace_bytes(b, s, h, n, d, code, cfg.causal))
    f_ms, b_ms, fb_ms = measure(lambda: tpmlp.tp_attn_flash_fwd(X, Wqkv, bqkv, Wo, QKV, LSE, O, Yp, ffws, **kw),
                         lambda: tpmlp.tp_attn_flash_bwd(dY, X, Wqkv, Wo, QKV, LSE, O, dQKV, dXp, dWqkv, dbqkv, dWo,
                                                         fbws, **kw))
    del ffws, fbws
    P = e(Z, s, s)
    mfws = u8(tpmlp.tp_attn_fwd_workspace_bytes(b, s, h, n, d, code, cfg.causal))
    mbws = u8(tpmlp.tp_attn_bwd_workspace_bytes(b, s, h, n, d, code, cfg.causal))
    mf_ms, mb_ms, mfb_ms = measure(lambda: tpmlp.tp_attn_fwd(X, Wqkv, bqkv, Wo, QKV, P, O, Yp, mfws, **kw),
                           lambda: tpmlp.tp_attn_bwd(dY, X, Wqkv, Wo, QKV, P, O, dQKV, dXp, dWqkv, dbqkv, dWo, mbws,
                                                     **kw))
    del P, mfws, mbws
    flops_f = 2.0 * T * h * 3 * q + 2.0 * T * q * h + 2 * 2.0 * Z * s * s * d * (0.5 if cfg.causal else 1.0)
    rate = lambda ms: 3 * flops_f / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg.dtype]
    tflops, m_tflops = rate(fb_ms), rate(mfb_ms)
    out = {"workload": f"{cfg.name}: one TP={cfg.tp} rank's attention of hidden {h}, {cfg.heads} heads of width {d} "
                       f"({n} on this rank), micro-batch {b} x seq {s}, causal, {cfg.dtype}",
           "path": "fused (tp_attn_flash_fwd + tp_attn_flash_bwd)",
           "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4), "fwd_bwd_ms": round(fb_ms, 4),
           "tflops": round(tflops, 2), "peak": peak,
           "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "bound": "mfma",
           "materialized": {"fwd_ms": round(mf_ms, 4), "bwd_ms": round(mb_ms, 4), "fwd_bwd_ms": round(mfb_ms, 4),
                            "tflops": round(m_tflops, 2),
                            "frac": round(m_tflops / peak, 4)},
           "cpu_baseline": None}
    return out


def attention_cpu(out):
    """The attention line's cpu_baseline: the float64 oracle on the same
    shard (forward, then a backward that recomputes the forward: 4 x the
    forward's work)."""
    import synth
    cfg = synth.get_attn_config("attn_2p4b")
    b, s, h, n, d = cfg.micro_batch, cfg.seq_len, cfg.hidden, cfg.heads_shard, cfg.head_dim
    inp = synth.draw_attn_inputs(b, s, h, n, d, cfg.dtype, seed=cfg.seed, sigma_dy=cfg.sigma_dy)
    T, q, Z = b * s, n * d, b * n
    flops_f = 2.0 * T * h * 3 * q + 2.0 * T * q * h + 2 * 2.0 * Z * s * s * d * (0.5 if cfg.causal else 1.0)
    out["cpu_baseline"] = attention_cpu_baseline(inp, cfg, 4 * flops_f)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="gpt_h10240")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the CPU oracle run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reuse", action="store_true",
                    help="skip the extra steps timed with the weight copies reused (profiled runs, so that every "
                         "step in the trace is a headline step)")
    ap.add_argument("--main-grad", action="store_true",
                    help="run the backward as tp_mlp_bwd_main_grad (dA, dB, db1 added to fp32 main gradients)")
    ap.add_argument("--recompute", action="store_true",
                    help="selective recomputation: the backward is tp_mlp_bwd_recompute (Z recomputed from X, the "
                         "forward's Z and H only scratch); value still counts the 12 T h f model flops")
    ap.add_argument("--b-transposed", action="store_true",
                    help="pass the second weight as B_i^T [hidden, ffn_shard] (TPMLP_LAYOUT_B_T); dB comes back "
                         "in that order")
    ap.add_argument("--no-reduce", action="store_true",
                    help="skip timing tp_mlp_reduce_partials (the TP group's sum of partials, not part of a step)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other MLP workloads (GPT-2-small, the 2.4B and 7B shards)")
    ap.add_argument("--no-attn", action="store_true",
                    help="skip timing the attention shard (fused and materialized paths, not part of a step)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before warm-up, run one plain device copy of this many MiB (a known-size kernel that "
                         "calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share (one TP rank) only: the path has no cross-GPU step here. "
              "Run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import megatron_tensor_transformer_04_amd as tpmlp

    tpmlp.load()
    cfg = synth.get_config(args.config)
    T, h, f = cfg.tokens, cfg.hidden, cfg.ffn_shard
    log(f"drawing inputs for {cfg.name} (T={T} h={h} f={f} {cfg.dtype})")
    inp = synth.draw_config(cfg)
    if cfg.all_shards:  # bench one rank's share
        import oracle
        inp.A, inp.b1, inp.B = (x.copy() for x in oracle.shard_weights(inp.A, inp.b1, inp.B, cfg.tp, 0))
        inp._bits.clear()
    from synth.device import device_inputs, torch_dtype
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    X, A, b1, B, dY = device_inputs(inp)
    td = torch_dtype(cfg.dtype)
    e = lambda *s: torch.empty(s, dtype=td, device=dev)
    Z, H, Yp = e(T, f), e(T, f), e(T, h)
    bt = args.b_transposed
    layout = tpmlp.TPMLP_LAYOUT_B_T if bt else 0
    if bt:
        B = B.t().contiguous()
    dZ, dXp, dA, dB, db1 = e(T, f), e(T, h), e(h, f), e(h, f) if bt else e(f, h), e(f)
    code = {"f32": tpmlp.TPMLP_F32, "f16": tpmlp.TPMLP_F16, "bf16": tpmlp.TPMLP_BF16}[cfg.dtype]
    nws = tpmlp.tp_mlp_workspace_bytes(T, h, f, code, 0, layout)
    ws = torch.empty((max(nws, 1),), dtype=torch.uint8, device=dev)
    nfws = tpmlp.tp_mlp_fwd_workspace_bytes(T, h, f, code, layout)
    fws = torch.empty((nfws,), dtype=torch.uint8, device=dev) if nfws else None
    log(f"workspace: forward {nfws / 2**20:.0f} MiB, backward {nws / 2**20:.0f} MiB")

    if args.main_grad:
        f32 = lambda *s: torch.zeros(s, dtype=torch.float32, device=dev)
        dA_main, dB_main, db1_main = f32(h, f), f32(h, f) if bt else f32(f, h), f32(f)

    if args.recompute:
        if args.main_grad:
            sys.exit("--recompute and --main-grad are separate entry points; pick one")
        nrws = tpmlp.tp_mlp_workspace_bytes(T, h, f, code, tpmlp.TPMLP_WS_RECOMPUTE, layout)
        rws = torch.empty((max(nrws, 1),), dtype=torch.uint8, device=dev)

    def step(fe=None, be=None, reuse=False):
        if args.recompute:
            # Z and H are scratch here (not kept for the backward, which recomputes them)
            tpmlp.tp_mlp_fwd(X, A, b1, B, Z, H, Yp, fws, events=fe, b_transposed=bt)
            tpmlp.tp_mlp_bwd_recompute(dY, X, A, b1, B, dZ, dXp, dA, dB, db1, rws, events=be, b_transposed=bt)
            return
        tpmlp.tp_mlp_fwd(X, A, b1, B, Z, H, Yp, fws, events=fe, b_transposed=bt, weights_staged=reuse)
        if args.main_grad:
            tpmlp.tp_mlp_bwd_main_grad(dY, X, A, B, Z, H, dZ, dXp, dA_main, dB_main, db1_main, ws, events=be,
                                       b_transposed=bt)
        else:
            tpmlp.tp_mlp_bwd(dY, X, A, B, Z, H, dZ, dXp, dA, dB, db1, ws, events=be, b_transposed=bt)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {n} bytes read and written by one copy kernel")
        del src, dst

    # The other MLP workloads and the attention shard first: each measured
    # from its own warm-up rather than right after the main workload's run
    # (whose power draw sets the clock the chip settles at). Their CPU
    # baselines come after the main timing.
    other = None
    if not args.no_configs and not (args.main_grad or args.recompute or bt):
        other = {n: config_rate(tpmlp, n, dev) for n in OTHER_CONFIGS if n != cfg.name}
    attn_line = None if args.no_attn else attention_rate(tpmlp, dev)
    torch.cuda.synchronize()

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    bwd_steps = (["rTA", "rF1"] + BWD_STEPS) if args.recompute else BWD_STEPS
    nf, nb = len(FWD_STEPS) + 1, len(bwd_steps) + 1
    mk = lambda: torch.cuda.Event(enable_timing=True)
    # Per-step breakdown (kernel_ms, the medians): K untimed steps with an event
    # at every step boundary. Each event record idles the stream for a few
    # microseconds, so the timed region below records only two per step.
    fev = [[mk() for _ in range(nf)] for _ in range(K)]
    bev = [[mk() for _ in range(nb)] for _ in range(K)]
    log(f"breakdown: {K} steps with every step boundary recorded")
    for k in range(K):
        step(fev[k], bev[k])
    torch.cuda.synchronize()
    per = {n: 0.0 for n in FWD_STEPS + bwd_steps}
    for k in range(K):
        for i, n in enumerate(FWD_STEPS):
            per[n] += fev[k][i].elapsed_time(fev[k][i + 1])
        for i, n in enumerate(bwd_steps):
            per[n] += bev[k][i].elapsed_time(bev[k][i + 1])
    per = {n: v / K for n, v in per.items()}
    fwd_each = [fev[k][0].elapsed_time(fev[k][nf - 1]) for k in range(K)]
    bwd_each = [bev[k][0].elapsed_time(bev[k][nb - 1]) for k in range(K)]
    step_each = sorted(a + b for a, b in zip(fwd_each, bwd_each))
    med = lambda v: sorted(v)[len(v) // 2]
    dom = max(GEMM_STEPS, key=lambda n: per[n])

    # Timed region: K steps; the events are the dominant GEMM's two step
    # boundaries (for the roofline) and one pair around the whole region. All
    # are created (recorded once) before the clock starts.
    in_fwd = dom in FWD_STEPS
    di = (FWD_STEPS if in_fwd else bwd_steps).index(dom)
    ta, tb = [mk() for _ in range(K)], [mk() for _ in range(K)]
    g0, g1 = mk(), mk()
    for ev in ta + tb + [g0, g1]:
        ev.record()
    torch.cuda.synchronize()

    def bracket(k):
        arr = [None] * (nf if in_fwd else nb)
        arr[di], arr[di + 1] = ta[k], tb[k]
        return arr

    log(f"timing {K} steps ({dom} bracketed)")
    t0 = time.perf_counter()
    g0.record()
    for k in range(K):
        if in_fwd:
            step(bracket(k), None)
        else:
            step(None, bracket(k))
    g1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("timed region done")
    gpu_ms = g0.elapsed_time(g1) / K
    dom_ms = sum(ta[k].elapsed_time(tb[k]) for k in range(K)) / K
    ms = wall / K * 1e3
    flops = 12.0 * T * h * f
    value = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg.dtype]
    gemm_flops = 2.0 * T * h * f
    achieved = gemm_flops / (dom_ms * 1e-3) / 1e12

    # Beside the headline (every step copies the weights): the same K steps
    # as later micro-batches of a gradient-accumulation step run them, the
    # forward reusing the weight copies that the steps above left in its
    # workspace (TPMLP_LAYOUT_WEIGHTS_STAGED).
    reuse_ms = None
    if not (args.recompute or args.no_reuse):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            step(reuse=True)
        torch.cuda.synchronize()
        reuse_ms = (time.perf_counter() - t0) / K * 1e3

    reduce_line = None if args.no_reduce else reduce_partials_rate(tpmlp, Yp, cfg, dev)
    if attn_line is not None and not args.no_cpu_baseline:
        attention_cpu(attn_line)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": workload_name(cfg) + ("; fp32 main-gradient accumulation" if args.main_grad else "")
                   + ("; Z recomputed in the backward (value counts the 12 T h f model flops)" if args.recompute
                      else "")
                   + ("; second weight passed as B_i^T [hidden, ffn_shard]" if bt else ""),
                   "tokens": T, "hidden": h, "ffn_shard": f, "tp": cfg.tp},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "peak_tflops": peak,
        "gpu_ms_per_step": round(gpu_ms, 4),
        "weights_reused": None if reuse_ms is None else {
            "ms_per_step": round(reuse_ms, 4), "tflops": round(flops / (reuse_ms * 1e-3) / 1e12, 2),
            "note": "later micro-batches of a gradient-accumulation step: the forward reuses the weight copies "
                    "already in its workspace (not the headline value)"},
        "step_ms_median": round(med(step_each), 4),
        "step_ms_min": round(step_each[0], 4),
        "fwd_ms_median": round(med(fwd_each), 4),
        "bwd_ms_median": round(med(bwd_each), 4),
        "kernel_ms": {n: round(v, 4) for n, v in per.items()},
        "roofline": {
            "kernel": dom,
            "bound": "mfma" if cfg.dtype != "f32" else "alu",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            # counters were taken in the default mode only
            "traffic": None if (args.main_grad or args.recompute or bt) else profiled_traffic(cfg.name, dom),
        },
        "cpu_baseline": None,
        "reduce_partials": reduce_line,
        "attention": attn_line,
        "configs": other,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
