#!/usr/bin/env python3
"""Benchmark of the FP8 delayed-scaling linear on one MI355X.

Workload (one "step" = every step of the hot path once): the FP8 MLP block
FC1 -> GeLU -> FC2 of a transformer layer, one GPU's share: 8192 tokens,
hidden 4096, FFN 14336, bf16 activations (0.1% outlier channels x50) and
weights, HYBRID formats (E4M3 forward, E5M2 gradients), delayed scaling with
an amax history of 1024 and the "max" algorithm.  Per step:
  forward  FC1: amax+cast-transpose X and W1, FP8 GEMM + GeLU epilogue -> H (bf16), Z
           FC2: amax+cast-transpose H and W2, FP8 GEMM -> Y (bf16)
  backward FC2: amax+cast-transpose dY (E5M2), dgrad -> dH (bf16), wgrad -> dW2 (fp32)
           FC1: GeLU backward fused into the amax+cast-transpose of dZ, dgrad -> dX, wgrad -> dW1
  update   one fp8_amax_scale_update over the 6 tensors' histories.
6 GEMMs of 2*8192*4096*14336 flop each = 5.77e12 flop per step.

Prints one JSON line.  `value` is TFLOP/s of the whole step (inputs resident
in HBM).  `roofline` is the GEMM kernel: algorithmic flop per launch over its
average launch time, measured with HIP events around each launch (recorded by
the library on the launch stream) during a second pass of the same steps,
against the dense FP8 matrix-core peak (5.0 PFLOP/s); beside it the fraction
of the f16 matrix-core ceiling the exact inner product runs on, and the peak
at the shader clock measured while the GEMMs ran.  `cpu_baseline` times the
CPU oracle on a 1024-token slice of the same step, plus the quantisation
tensor in full, the 768-wide linear's steps and a slice of the layer's GEMMs.

`quant` times the standalone quantisation kernels on a 2^28-element bf16
tensor: amax alone, the dual-format amax+cast+transpose with the two metas'
scale update in its last workgroup, and dequant, in GB/s of algorithmic bytes,
beside streaming read and copy kernels of the same size.

`layer_step` reports the FP8 transformer-layer training step beside it: the
QKV, attention-output, FC1 and FC2 linears (hidden 8192, FFN 28672, 8192
tokens) forward and backward from fp32 master weights, around the bf16
attention core (64 heads of 128, 2 sequences of 4096 tokens), with dynamic
loss scaling and SGD, 20 iterations with the x100 input spike at iteration
10: 12 GEMMs (3.63e13 flop) and 3.30e12 flop of attention products per step.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, HID, FFN, HIST = 8192, 4096, 14336, 1024
GEMM_FLOP = 2.0 * M * HID * FFN
STEP_FLOP = 6 * GEMM_FLOP
PEAK_F16_TFLOPS = 2500.0      # MI355X dense f16/bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_CLOCK_MHZ = 2400.0       # the engine clock the peaks are quoted at


def mfma_roofline(tflops, avg_ms, per_launch_flop, clock_mhz, kernel, f16_inner):
    """The roofline object of a GEMM kernel against the dense FP8 matrix-core
    peak; the exact inner product also reports its f16 matrix-core ceiling,
    and both the peak at the shader clock measured while the GEMMs ran."""
    r = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
         "frac": round(tflops / PEAK_FP8_TFLOPS, 4), "traffic": None, "kernel": kernel,
         "per_launch_flop": per_launch_flop, "avg_launch_ms": round(avg_ms, 4)}
    if f16_inner:
        r["f16_ceiling"] = {"peak": PEAK_F16_TFLOPS, "frac": round(tflops / PEAK_F16_TFLOPS, 4),
                            "note": "the exact inner product runs on the f16 matrix cores (FP8 codes decoded to f16)"}
    if clock_mhz:
        ratio = clock_mhz / PEAK_CLOCK_MHZ
        ceiling = (PEAK_F16_TFLOPS if f16_inner else PEAK_FP8_TFLOPS) * ratio
        r["clock_mhz_measured"] = round(clock_mhz, 1)
        r["peak_at_measured_clock"] = round(PEAK_FP8_TFLOPS * ratio, 1)
        r["frac_at_measured_clock"] = round(tflops / (PEAK_FP8_TFLOPS * ratio), 4)
        if f16_inner:
            r["f16_ceiling"]["peak_at_measured_clock"] = round(ceiling, 1)
            r["f16_ceiling"]["frac_at_measured_clock"] = round(tflops / ceiling, 4)
    return r


def measure_clock(F, torch, run, window_ms):
    """Shader clock while `run()` enqueues GPU work: the library's clock
    sample runs on a stream of its own for window_ms after the work is
    enqueued."""
    clk = F.ClockSample()
    torch.cuda.synchronize()
    run()
    clk.start(int(window_ms * 1000))
    mhz = clk.mhz()
    torch.cuda.synchronize()
    return mhz


def _exit_multi_gpu(n):
    print(f"bench.py runs on one GPU only (asked for {n}): the library has no multi-GPU path.",
          file=sys.stderr, flush=True)
    sys.exit(2)


class MlpBlock:
    """The benchmark's MLP block on the seeded inputs (see synth.mlp_inputs)."""

    def __init__(self, F, torch, fast_accum=False):
        import synth
        from fp8_mixed_precision_reduce_amd.blocks import Fp8MlpBlock
        x, w1, w2, dy = synth.mlp_inputs(0, device="cuda")
        self.block = Fp8MlpBlock(x, w1, w2, dy, history_len=HIST, fast_accum=fast_accum)

    def step(self):
        self.block.step()

    @staticmethod
    def cast_bytes_per_step():
        """Algorithmic HBM bytes of the cast kernels in one step."""
        ct = lambda r, c: r * c * (2 + 2)          # read bf16, write codes and transposed codes
        return (ct(M, HID) + ct(FFN, HID) + ct(M, FFN) + ct(HID, FFN) + ct(M, HID)
                + M * FFN * (2 + 2 + 2))           # dgelu: read dH and Z, write codes twice


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_mlp_step_traffic.md")
GEMM_SOURCES = ("gemm.hip", "common.h")


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "fp8_mixed_precision_reduce_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def gemm_traffic():
    """HBM bytes per GEMM launch of the MLP step from the committed byte-counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter read for
    a plain copy of known size), or None when the GEMM sources have changed since
    the counters were taken (or no summary exists)."""
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    kv = dict(re.findall(r"^(\w+): (\S+)$", text, flags=re.M))
    if kv.get("gemm_source_sha256") != gemm_source_hash() or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


def time_steps(block, torch, steps, median=False):
    """Mean ms per step over `steps` steps (events at every step boundary);
    with median=True also the median step."""
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        block.step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    mean = ev[0].elapsed_time(ev[steps]) / steps
    if not median:
        return mean
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return mean, per[steps // 2]


def kernel_breakdown(block, F, torch, steps):
    """Per-kind launch times over `steps` further steps (HIP events recorded
    by the library around each of its launches, on the launch stream)."""
    F.timing_enable(64 * steps)
    torch.cuda.synchronize()
    for _ in range(steps):
        block.step()
    torch.cuda.synchronize()
    rec = F.timing_read(64 * steps)
    F.timing_enable(0)
    out = {}
    for kind, ms in rec:
        n, tot = out.get(kind, (0, 0.0))
        out[kind] = (n + 1, tot + ms)
    return out


def layer_leg(F, torch, fast_accum=False, iterations=20, breakdown_steps=3):
    """The transformer-layer step: per-iteration times over the run with the
    spike, then a per-kind kernel breakdown over a few further steps."""
    import synth
    from fp8_mixed_precision_reduce_amd.blocks import Fp8TransformerLayer
    cfg = synth.LAYER
    inp = synth.layer_inputs(device="cuda")
    lay = Fp8TransformerLayer(inp["x"], None, inp["g"], None, inp["wqkv"], inp["wo"], inp["w1"], inp["w2"],
                              history_len=cfg["history_len"], fast_accum=fast_accum, heads=cfg["heads"],
                              batch=cfg["batch"])
    for k in ("wqkv", "wo", "w1", "w2", "ctx", "dqkv"):
        del inp[k]                                        # copied into the layer's master buffer
    spiked = synth.layer_spike(inp["x"], cfg["spike_factor"])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iterations + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(iterations):
        lay.step(spiked if i == cfg["spike_iteration"] else None)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per_it = [ev[i].elapsed_time(ev[i + 1]) for i in range(iterations)]
    state = lay.ls_state.cpu().tolist()
    F.timing_enable(96 * breakdown_steps)
    torch.cuda.synchronize()
    for _ in range(breakdown_steps):
        lay.step()
    torch.cuda.synchronize()
    rec = F.timing_read(96 * breakdown_steps)
    F.timing_enable(0)
    kb = {}
    for kind, ms in rec:
        n, tot = kb.get(kind, (0, 0.0))
        kb[kind] = (n + 1, tot + ms)
    flop = lay.flops_per_step()
    attn_flop = lay.attention_flops()
    gemm_flop = flop - attn_flop
    n_params = lay.master.numel()
    later = sorted(per_it[2:])
    mean_ms = sum(per_it[2:]) / len(per_it[2:])
    n_sgd, t_sgd = kb.get("sgd", (0, 0.0))
    sgd_ms = t_sgd / n_sgd if n_sgd else float("nan")
    sgd_step_ms = t_sgd / breakdown_steps
    sgd_bytes = (14 if lay.fuse_sgd_cast else 12) * n_params
    mhz = measure_clock(F, torch, lambda: [lay.step() for _ in range(3)], 1.5 * mean_ms)
    n_g, t_g = kb.get("gemm", (1, float("nan")))
    gemm_tflops = gemm_flop * breakdown_steps / (t_g * 1e-3) / 1e12
    attn_ms = kb.get("attention", (0, float("nan")))[1] / breakdown_steps
    attn_tflops = attn_flop / (attn_ms * 1e-3) / 1e12
    out = {
        "workload": "FP8 transformer layer step: QKV, attention-out, FC1, FC2 linears fwd+bwd around the bf16 "
                    "attention core (64 heads of 128, seq 4096 x batch 2, no mask), hidden 8192, FFN 28672, "
                    "tokens 8192, fp32 masters + SGD + dynamic loss scaling, x100 spike at iteration 10, "
                    "history 1024",
        "iterations": iterations,
        "ms_per_step_mean_2_to_end": round(mean_ms, 4),
        "ms_per_step_median": round(later[len(later) // 2], 4),
        "ms_spike_iteration": round(per_it[cfg["spike_iteration"]], 4),
        "tflops": round(flop / (mean_ms * 1e-3) / 1e12, 2),
        "flop_per_step": flop,
        "loss_scale_after": state[0],
        "kernels_ms_per_step": {k: round(v[1] / breakdown_steps, 4) for k, v in sorted(kb.items())},
        "roofline": mfma_roofline(gemm_tflops, t_g / n_g, gemm_flop / 12, mhz,
                                  "k_gemm, the step's 12 FP8 GEMM calls (QKV, O, FC1, FC2 fprop, dgrad and wgrad); "
                                  "achieved = their algorithmic flop over their summed event time",
                                  not fast_accum),
        "attention": {"flop_per_step": attn_flop,
                      "ms_per_step": round(attn_ms, 4),
                      "tflops": round(attn_tflops, 1),
                      "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_F16_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_F16_TFLOPS, 4),
                                   "traffic": None, "kernel": "k_attn_fwd, k_attn_bwd_kv, k_attn_bwd_q (bf16 MFMA)",
                                   "peak_at_measured_clock": round(PEAK_F16_TFLOPS * mhz / PEAK_CLOCK_MHZ, 1)},
                      "note": "forward (QK^T, PV) and backward (dP, dV, dQ, dK) products over the attention "
                              "kernels' event time; the transposes into the workspaces are under 'other'"},
        "sgd": {"params": n_params, "fused_with_weight_cast": lay.fuse_sgd_cast,
                "launches_per_step": n_sgd // breakdown_steps, "avg_launch_ms": round(sgd_ms, 4),
                "ms_per_step": round(sgd_step_ms, 4), "bytes_per_step": sgd_bytes,
                "achieved_gbs": round(sgd_bytes / (sgd_step_ms * 1e-3) / 1e9, 1), "peak_gbs": PEAK_HBM_GBS,
                "frac": round(sgd_bytes / (sgd_step_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "note": "fused: fp8_sgd_step_cast per weight matrix (master read and written, gradient read, E4M3 "
                        "codes written row-major and transposed: 14 B per parameter), the next forward taking W "
                        "pre-cast; unfused: fp8_sgd_step over all masters (12 B per parameter)"},
    }
    del lay, inp, spiked
    torch.cuda.empty_cache()
    return out


def linear768_leg(F, torch, iters=200, steps_per_graph=20):
    """The 768-wide linear (1024 x 768 x 768, fp32 in and out, history 16): one
    forward step (amax + cast of X and W, FP8 GEMM with bias, scale update) and
    one forward + backward step in HYBRID (adds the E5M2 cast-transpose of dY,
    dgrad and wgrad), each timed launched one call at a time (eager) and
    replayed from a captured HIP graph of `steps_per_graph` consecutive steps
    (one replay launches them all; a graph of a single step would time the
    graph launch itself, which costs more than the step's few small kernels).
    At 1.2 GFLOP per GEMM these steps are bound by launch latency, not by the
    matrix cores or HBM, so they are reported in microseconds per step."""
    import synth
    m, n, k = 1024, 768, 768
    w, b = (t.cuda() for t in synth.linear768_weights())
    x, dy = synth.linear768_x(0).cuda(), synth.linear768_dy(0).cuda()
    recipe = F.Recipe(F.FORMAT_HYBRID, 16, F.AMAX_MAX, 0)
    bank = F.MetaBank([F.E4M3, F.E4M3, F.E5M2], 16, device="cuda")
    saved = F.Saved(m, n, k, device="cuda")
    y = torch.empty(m, n, device="cuda")
    dx, dw = torch.empty(m, k, device="cuda"), torch.empty(n, k, device="cuda")
    gq, gqt = torch.empty(m, n, dtype=torch.uint8, device="cuda"), torch.empty(n, m, dtype=torch.uint8, device="cuda")

    def fwd():
        F.fp8_linear_fwd(x, w, y, recipe, bank.meta(0), bank.meta(1), saved, bias=b)
        bank.update(recipe)

    def fwd_bwd():
        F.fp8_linear_fwd(x, w, y, recipe, bank.meta(0), bank.meta(1), saved, bias=b)
        F.fp8_linear_bwd(dy, k, recipe, bank.meta(2), saved, gq, gqt, dx, dw)
        bank.update(recipe)

    def timed(fn, calls, batches=5):
        # median over batches of `calls` calls (us per call): a one-off stall (a
        # clock change, the first replay's upload) does not move the figure
        per = []
        for _ in range(batches):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            for _ in range(calls):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            per.append(ev[0].elapsed_time(ev[1]) * 1e3 / calls)
        return sorted(per)[batches // 2]

    out = {"workload": "linear 1024x768x768 fp32 in/out, E4M3 (forward) / HYBRID (forward+backward), "
                       "history 16, launch-latency bound", "iterations": iters, "steps_per_graph": steps_per_graph,
           "statistic": "median over 5 batches of iterations / 5 steps (graph: replays of steps_per_graph "
                        "steps, per step)"}
    for name, fn in (("forward", fwd), ("forward_backward", fwd_bwd)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        eager = timed(fn, iters // 5)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps_per_graph):
                fn()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        graph = timed(g.replay, max(1, iters // (5 * steps_per_graph))) / steps_per_graph
        out[name] = {"us_per_step_eager": round(eager, 2), "us_per_step_graph": round(graph, 2)}
        del g
    return out


def quant_leg(F, torch, reps=50, first=10):
    """Standalone quantisation of the 2^28-element bf16 tensor (16384 x 16384,
    row magnitudes 2^u, u ~ U[-20, 10]), `reps` repetitions on the same tensor:
    (i) amax alone, (ii) one dual-format cast-transpose (amax fused, E4M3 and
    E5M2, both layouts) whose last workgroup runs the scale update of the two
    metas, (iii) dequant of both code tensors back to bf16; beside them the
    streaming read and copy kernels over the same 512 MiB (the HBM rate this
    layout reaches without arithmetic).  Per-kernel times from the library's
    launch events; mean (and median) over repetitions `first`..reps-1."""
    import synth
    cfg = synth.QUANT
    rows, cols, L = cfg["rows"], cfg["cols"], cfg["history_len"]
    n = rows * cols
    x = synth.quant_tensor(device="cuda")
    bank = F.MetaBank([F.E4M3, F.E5M2], L)
    recipe = F.Recipe(F.FORMAT_HYBRID, L, F.AMAX_MAX, 0)
    ticket = torch.zeros(1, dtype=torch.int32, device="cuda")
    slot = torch.zeros(1, dtype=torch.float32, device="cuda")
    u8 = dict(dtype=torch.uint8, device="cuda")
    q4, q4t, q5, q5t = (torch.empty(rows, cols, **u8), torch.empty(cols, rows, **u8), torch.empty(rows, cols, **u8),
                        torch.empty(cols, rows, **u8))
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty(2, rows, cols, dtype=torch.bfloat16, device="cuda")
    words = torch.empty(4096, dtype=torch.int32, device="cuda")
    seq = [("amax", lambda: F.fp8_amax(x, slot)),
           ("cast_transpose_dual_update", lambda: F.fp8_cast_transpose_dual_update(x, bank, recipe, ticket,
                                                                                   q4, q4t, q5, q5t)),
           ("dequant_both", lambda: (F.fp8_dequant(q4, F.E4M3, bank.scale_inv[0:1], out),
                                     F.fp8_dequant(q5, F.E5M2, bank.scale_inv[1:2], out)))]
    ceil = [("stream_read", lambda: F.stream_probe(x, words, 0)), ("stream_copy", lambda: F.stream_probe(x, out, 1)),
            ("stream_copy_nt", lambda: F.stream_probe(x, out, 2)),
            ("stream_copy_twice", lambda: F.stream_probe(x, out2, 3)),
            ("stream_copy_twice_nt", lambda: F.stream_probe(x, out2, 4))]
    nbytes = {"amax": 2 * n, "cast_transpose_dual_update": (2 + 4) * n, "dequant_both": 2 * (1 + 2) * n,
              "stream_read": 2 * n, "stream_copy": 2 * 2 * n, "stream_copy_nt": 2 * 2 * n,
              "stream_copy_twice": 3 * 2 * n, "stream_copy_twice_nt": 3 * 2 * n}

    def launches():
        rec = F.timing_read(16 * reps)
        F.timing_enable(0)
        return [ms for _, ms in rec]

    def stat(v, nb):
        mean = sum(v) / len(v)
        med = sorted(v)[len(v) // 2]
        return {"mean_ms": round(mean, 4), "median_ms": round(med, 4), "bytes": nb,
                "achieved_gbs": round(nb / (mean * 1e-3) / 1e9, 1),
                "frac": round(nb / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}

    # (1) the configuration's sequence: per repetition amax, the fused cast-transpose
    # with the update, dequant of both; per-kernel times from the library's events
    F.timing_enable(16 * reps)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for r in range(reps):
        for _, fn in seq:
            fn()
        ev[r + 1].record()
    torch.cuda.synchronize()
    v = launches()
    per_rep = [ev[r].elapsed_time(ev[r + 1]) for r in range(first, reps)]
    per = {"amax": v[0::4][first:], "cast_transpose_dual_update": v[1::4][first:],
           "dequant_both": [a + b for a, b in zip(v[2::4], v[3::4])][first:]}
    res = {
        "workload": "bf16 16384x16384 (2^28 elements), row magnitudes 2^u, u~U[-20,10]; "
                    f"{reps} repetitions, mean of {first}..{reps - 1}",
        "sequence_ms_per_repetition": round(sum(per_rep) / len(per_rep), 4),
    }
    for k in per:
        res[k] = stat(per[k], nbytes[k])
    # (2) each kernel back to back with itself (its own write-backs included),
    # beside the streaming read and copy kernels measured the same way
    steady = {}
    for name, fn in seq + ceil:
        for _ in range(3):
            fn()
        F.timing_enable(16 * reps)
        torch.cuda.synchronize()
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        w = launches()
        if name == "dequant_both":
            w = [a + b for a, b in zip(w[0::2], w[1::2])]
        steady[name] = stat(w, nbytes[name])
    copy_ceiling = max(steady["stream_copy"]["achieved_gbs"], steady["stream_copy_nt"]["achieved_gbs"])
    twice_ceiling = max(steady["stream_copy_twice"]["achieved_gbs"], steady["stream_copy_twice_nt"]["achieved_gbs"])
    for k in ("amax", "cast_transpose_dual_update", "dequant_both"):
        # the ceiling of the same read:write ratio: read only for amax, one read
        # and two writes for the dual cast (2 B in, 4 B out) and the dequant (1 B in,
        # 2 B out); the 1:1 copy beside it
        ceiling = steady["stream_read"]["achieved_gbs"] if k == "amax" else twice_ceiling
        steady[k]["frac_of_stream_ceiling"] = round(steady[k]["achieved_gbs"] / ceiling, 4)
        if k != "amax":
            steady[k]["frac_of_copy_ceiling"] = round(steady[k]["achieved_gbs"] / copy_ceiling, 4)
    res["steady_state"] = steady
    res["peak_gbs"] = PEAK_HBM_GBS
    res["note"] = ("cast_transpose_dual_update: amax + cast to E4M3 and E5M2 + both transposes + the two metas' "
                   "scale update (last workgroup), one launch.  steady_state: each kernel 20 times back to back; "
                   "stream_read / stream_copy(_nt) / stream_copy_twice(_nt): the same 16-byte load/store layout with "
                   "no arithmetic (the copies with plain or non-temporal stores, the twice variants writing every "
                   "vector to two places); frac_of_stream_ceiling is against the pattern of the same read:write "
                   "ratio (read for amax, the faster copy-twice for the dual cast-transpose and the dequant), "
                   "frac_of_copy_ceiling against the faster 1:1 copy")
    del x, q4, q4t, q5, q5t, out, out2
    torch.cuda.empty_cache()
    return res


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo, with its family and model
    numbers (a virtualised host may report only a generic name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break                      # the first processor's block is enough
                key, _, val = line.partition(":")
                fields.setdefault(key.strip(), val.strip())
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    extra = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
    return f"{name} ({extra})" if extra else name


def cpu_baseline(torch, rows=1024, layer_rows=32):
    """The CPU oracle, as it stands, on the host cores: (value) a `rows`-token
    slice of the MLP block step; beside it the quantisation tensor in full,
    the 768-wide linear's forward and forward+backward steps in full (median
    of 5), and `layer_rows` output rows of each of the transformer layer's
    12 GEMMs (extrapolated to the full step, and labelled so)."""
    import numpy as np

    import oracle as O
    import synth
    x, w1, w2, dy = synth.mlp_inputs(0, device="cuda")
    to16 = lambda t: t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    xs, dys, w1n, w2n = to16(x[:rows]), to16(dy[:rows]), to16(w1), to16(w2)
    del x, w1, w2, dy
    t0 = time.perf_counter()
    O.mlp_step(xs, w1n, w2n, dys, O.mlp_metas(HIST))
    dt = time.perf_counter() - t0
    flop = 6 * 2.0 * rows * HID * FFN
    del xs, dys, w1n, w2n
    legs = {}
    # the quantisation tensor, in full: amax, the cast-transpose to both formats
    # with the update, dequant of both
    xq = to16(synth.quant_tensor(device="cuda"))
    n = xq.size
    metas = [O.Meta(synth.QUANT["history_len"], 0), O.Meta(synth.QUANT["history_len"], 1)]
    t0 = time.perf_counter()
    O.amax(xq)
    ta = time.perf_counter() - t0
    t0 = time.perf_counter()
    codes = [O.cast_transpose(xq, f, metas[f].scale)[0] for f in (0, 1)]
    for m in metas:
        m.record(xq)
    O.update_metas(metas)
    tc = time.perf_counter() - t0
    t0 = time.perf_counter()
    for f in (0, 1):
        O.dequant(codes[f], f, metas[f].scale_inv, 1)
    td = time.perf_counter() - t0
    del xq, codes
    legs["quant_full"] = {"sample": "the 2^28-element bf16 tensor in full (one repetition)",
                          "amax_gbs": round(2 * n / ta / 1e9, 3),
                          "cast_transpose_dual_update_gbs": round(6 * n / tc / 1e9, 3),
                          "dequant_both_gbs": round(6 * n / td / 1e9, 3),
                          "seconds": round(ta + tc + td, 2)}
    # the 768-wide linear, in full
    w, b = synth.linear768_weights()
    xl, dyl = synth.linear768_x(0).numpy(), synth.linear768_dy(0).numpy()
    w, b = w.numpy(), b.numpy()

    def med5(fn):
        t = []
        for _ in range(5):
            t0 = time.perf_counter()
            fn()
            t.append(time.perf_counter() - t0)
        return sorted(t)[2]

    def fwd():
        return O.linear_fwd(xl, w, O.Meta(16, 0), O.Meta(16, 0), bias=b)

    tf = med5(fwd)
    tfb = med5(lambda: O.linear_bwd(dyl, fwd(), O.Meta(16, 1)))
    legs["linear768"] = {"sample": "1024x768x768 linear, one step in full, median of 5",
                         "forward_ms": round(tf * 1e3, 3), "forward_backward_ms": round(tfb * 1e3, 3),
                         "forward_gflops": round(2.0 * 1024 * 768 * 768 / tf / 1e9, 2),
                         "forward_backward_gflops": round(3 * 2.0 * 1024 * 768 * 768 / tfb / 1e9, 2)}
    # the transformer layer's 12 GEMMs on `layer_rows` output rows each
    cfg = synth.LAYER
    m_, h_, f_ = cfg["m"], cfg["hidden"], cfg["ffn"]
    shapes = [(m_, 3 * h_, h_), (m_, h_, h_), (m_, f_, h_), (m_, h_, f_),          # fprop
              (m_, h_, 3 * h_), (m_, h_, h_), (m_, h_, f_), (m_, f_, h_),          # dgrad
              (3 * h_, h_, m_), (h_, h_, m_), (f_, h_, m_), (h_, f_, m_)]          # wgrad
    rng = np.random.default_rng(0)
    big = rng.integers(0, 0x77, max(n_ * k_ for _, n_, k_ in shapes), dtype=np.uint8)
    a_rows = rng.integers(0, 0x77, layer_rows * max(k_ for _, _, k_ in shapes), dtype=np.uint8)
    t_slice, flop_slice, flop_full = 0.0, 0.0, 0.0
    for mm, nn, kk in shapes:
        a = a_rows[:layer_rows * kk].reshape(layer_rows, kk)
        bmat = big[:nn * kk].reshape(nn, kk)
        t0 = time.perf_counter()
        O.gemm(a, 0, bmat, 0)
        t_slice += time.perf_counter() - t0
        flop_slice += 2.0 * layer_rows * nn * kk
        flop_full += 2.0 * mm * nn * kk
    legs["layer_gemms_slice"] = {
        "sample": f"the transformer layer's 12 GEMMs, {layer_rows} output rows each (operand codes drawn at random: "
                  "the oracle's GEMM time does not depend on the values)",
        "gflops": round(flop_slice / t_slice / 1e9, 2), "seconds": round(t_slice, 2),
        "extrapolated_full_step_s": round(t_slice * flop_full / flop_slice, 1),
        "extrapolated": True}
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": O.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"MLP block fwd+bwd+update on {rows} of {M} tokens (hidden {HID}, FFN {FFN}, full "
                      f"weights, history {HIST}); {dt:.2f} s for {flop:.3g} flop",
            "legs": legs}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fast-accum", action="store_true", help="time the fast-accumulation GEMMs as the main value")
    ap.add_argument("--no-layer", action="store_true", help="skip the transformer-layer step")
    ap.add_argument("--no-quant", action="store_true", help="skip the standalone quantisation kernels")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="first run a plain elementwise copy (torch.neg) of GIB GiB of fp32 three times, as the "
                         "known-size reference kernel for hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        _exit_multi_gpu(args.gpus)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        _exit_multi_gpu(int(os.environ["WORLD_SIZE"]))

    import torch

    import fp8_mixed_precision_reduce_amd as F

    t0 = time.perf_counter()

    def progress(what):
        print(f"bench: {what} done ({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)

    if args.copy_calibration > 0:
        n = int(args.copy_calibration * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    block = MlpBlock(F, torch, fast_accum=args.fast_accum)
    for _ in range(args.warmup):
        block.step()
    ms, ms_median = time_steps(block, torch, args.steps, median=True)
    kb = kernel_breakdown(block, F, torch, args.steps)
    progress("MLP block step")
    n_g, t_g = kb.get("gemm", (1, float("nan")))
    gemm_ms = t_g / n_g
    gemm_tflops = GEMM_FLOP / (gemm_ms * 1e-3) / 1e12
    cast_ms = sum(kb.get(k, (0, 0.0))[1] for k in ("cast_transpose", "cast")) / args.steps
    cast_gbs = MlpBlock.cast_bytes_per_step() / (cast_ms * 1e-3) / 1e9

    mhz = measure_clock(F, torch, lambda: [block.step() for _ in range(10)], 5 * ms)
    progress("shader clock under the MLP step")

    # the other accumulation mode, for reference, with its own GEMM roofline
    other = MlpBlock(F, torch, fast_accum=not args.fast_accum)
    for _ in range(2):
        other.step()
    other_ms = time_steps(other, torch, max(3, args.steps // 2))
    kb_o = kernel_breakdown(other, F, torch, max(3, args.steps // 2))
    n_o, t_o = kb_o.get("gemm", (1, float("nan")))
    other_mhz = measure_clock(F, torch, lambda: [other.step() for _ in range(10)], 5 * other_ms)
    other_roof = mfma_roofline(GEMM_FLOP / (t_o / n_o * 1e-3) / 1e12, t_o / n_o, GEMM_FLOP, other_mhz,
                               "k_gemm (fp8 GEMM, 256x256 tiles), " + ("exact" if args.fast_accum else "fast") +
                               " inner product", args.fast_accum)
    del other

    # just-in-time scaling (every cast preceded by its own amax pass), for reference
    block.block.recipe.just_in_time = 1
    for _ in range(2):
        block.step()
    jit_ms = time_steps(block, torch, max(3, args.steps // 2))
    block.block.recipe.just_in_time = 0
    torch.cuda.empty_cache()
    progress("other accumulation mode and just-in-time scaling")
    lin768 = linear768_leg(F, torch)
    progress("768-wide linear")
    layer = None if args.no_layer else layer_leg(F, torch, fast_accum=args.fast_accum)
    if layer is not None:
        progress("transformer-layer step")
    quant = None if args.no_quant else quant_leg(F, torch)
    if quant is not None:
        progress("quantisation kernels")

    value = STEP_FLOP / (ms * 1e-3) / 1e12
    roofline = mfma_roofline(gemm_tflops, gemm_ms, GEMM_FLOP, mhz, "k_gemm (fp8 GEMM, 256x256 tiles), " +
                             ("fast" if args.fast_accum else "exact") + " inner product", not args.fast_accum)
    roofline["traffic"] = gemm_traffic()
    line = {
        "metric": "FP8 linear fwd+bwd TFLOP/s (% FP8 MFMA peak); cast/amax GB/s (% HBM)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_median, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {
            "workload": "FP8 MLP block fwd+bwd (FC1-GeLU-FC2), tokens 8192, hidden 4096, FFN 14336, HYBRID "
                        "E4M3/E5M2, delayed scaling, amax history 1024, max",
            "global_batch": M, "hidden": HID, "ffn": FFN, "history_len": HIST,
            "gemm_inner_product": "fast: native fp8 MFMA" if args.fast_accum
            else "exact: fp8 codes decoded to f16, f16 MFMA, fp32 accumulation",
            "frac_of_fp8_peak": round(value / PEAK_FP8_TFLOPS, 4),
        },
        "roofline": roofline,
        "kernels_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in sorted(kb.items())},
        "cast_kernels": {"achieved_gbs": round(cast_gbs, 1), "peak_gbs": PEAK_HBM_GBS,
                         "frac": round(cast_gbs / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes_per_step": MlpBlock.cast_bytes_per_step()},
        ("exact_accum" if args.fast_accum else "fast_accum"): {
            "ms_per_step": round(other_ms, 4), "tflops": round(STEP_FLOP / (other_ms * 1e-3) / 1e12, 2),
            "roofline": other_roof},
        "just_in_time_scaling": {
            "ms_per_step": round(jit_ms, 4), "tflops": round(STEP_FLOP / (jit_ms * 1e-3) / 1e12, 2),
            "note": "same step with every tensor scaled from its own current amax (an extra amax pass each)"},
    }
    line["linear768"] = lin768
    if layer is not None:
        line["layer_step"] = layer
    if quant is not None:
        line["quant"] = quant
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(torch)
        progress("oracle on the host")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
