"""Benchmark of the POET-X linear layer (fwd + bwd) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--gpus 1]

One step = Cayley build of R and P (one launch set for both), forward and
backward (to x and to the generators, including the Cayley VJP) of every
layer of the workload, with all inputs resident in HBM. The default workload
is the 8B-class MLP up-projection: W0 14336 x 4096 (out x in), b = 256,
8192 tokens, bf16 storage with float32 accumulation.

Order of work: the float64 oracle on the host's cores (a bounded token
sample, timed before any GPU timing), W warm-up steps, K instrumented steps
for the per-stage breakdown (untimed for `value`; they also bring the GPU's
clock back up after the oracle's idle seconds), K timed steps (mean and
median per step), K "cold" steps each after a 512 MB scratch write that
evicts the Infinity Cache, then a sampled parity check of every layer
against the oracle.

Prints ONE JSON line: tokens/s of the whole step, the roofline of the
dominant kernel (the dense W0 GEMM of the forward, timed live with HIP events
on the launch stream), the layer's algorithmic roofline fraction, the cold
variant, the parity sample and the oracle's own throughput.

Each event record puts a few microseconds between two kernels, so the timed
steps hold only an event at every step boundary and the pair around the
dominant kernel; the per-stage breakdown (stages_ms, instrumented_step_ms)
comes from as many further steps with an event pair around every stage.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "POET-X linear fwd+bwd tokens/s at 8B-shaped layer; % bf16 MFMA roofline"
PEAK_BF16 = 2516.6e12   # MI355X dense bf16 MFMA, FLOP/s
PEAK_F32 = 157.3e12     # MI355X fp32 (matrix), FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E, B/s

# stage names by the library's stage index (None: a stage that does not run)
FWD_STAGES = ["p_apply", "dense_fwd", "r_apply"]
FWD_PERM_STAGES = ["gather_x", "scatter_y"]
FWD_INT8_STAGE = 5       # widen the INT8 codes, scale R's block columns
BWD_INT8_STAGE = 10
# Where a side's gradient apply and gram share one launch (bf16, b = 32-256),
# grad_r / grad_x time that launch and gram_r / gram_p the gram's reduction.
BWD_STAGES = ["grad_r", "gram_r", "dense_bwd", "gram_p", "grad_x", "vjp_r", "vjp_p"]
BWD_PERM_STAGES = ["gather_gy_x", "scatter_gx"]


def layer_work(s, saved_y=False):
    """Algorithmic flops and bytes of one layer's step (build + fwd + bwd).
    The forward writes y and Z, or y alone when y is kept in Z's place."""
    N, n, m, b = s.tokens, s.d_in, s.d_out, s.b
    es = 2 if s.dtype == "bf16" else 4
    flops = 4 * N * m * n + 6 * N * b * (m + n) + 6 * b * b * (m + n)
    blocks = b * (m + n)          # elements of all R and P blocks
    theta = (m + n) * (b - 1) // 2
    fwd = es * (N * n + m * n + blocks + (1 if saved_y else 2) * N * m) + 4 * theta
    bwd = es * (2 * N * m + N * n + m * n + blocks + N * n) + 4 * blocks + 4 * theta
    build = 4 * theta + 4 * blocks + es * blocks
    return flops, fwd + bwd + build


def cpu_baseline(spec, sample_tokens, map="cayley", permute=False, int8=False):
    """The float64 oracle (build, materialise, forward, backward) on the first
    `sample_tokens` tokens of the workload, timed on the host's cores."""
    import dataclasses

    import oracle.poetx_oracle as O
    from orthogonal_equivalence_amd.inputs import make_layer, make_permutations
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max(i.get("num_threads", 1) for i in info) if info else 1
        if info:
            i = info[0]
            blas = (f"{i.get('internal_api', '?')} {i.get('version', '?')} "
                    f"({os.path.basename(i.get('filepath', '?'))}, {i.get('num_threads', '?')} threads)")
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    L = make_layer(spec)
    x, g_y = L.x[:sample_tokens], L.g_y[:sample_tokens]
    # repeat the whole oracle step until about 10 s of CPU work (at most 6 reps)
    reps, t0 = 0, time.perf_counter()
    while True:
        po, pi = make_permutations(spec) if permute else (None, None)
        W0 = O.dequantize_rows(*O.quantize_rows(L.W0)) if int8 else L.W0
        ora = O.LayerOracle(W0, L.theta_R, L.theta_P, spec.b, spec.b, map=map, perm_out=po,
                            perm_in=pi)
        ora.forward(x)
        ora.backward(g_y, x)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 6:
            break
    return {"value": reps * sample_tokens / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas": blas, "timed": "before the GPU timing, same process",
            "sample": f"{reps} float64 oracle steps (exact Cayley solves, block-local "
                      f"materialisation of R W0 P, forward, backward) on the first "
                      f"{sample_tokens} of {spec.tokens} tokens of {spec.name} "
                      f"{spec.d_out}x{spec.d_in} b={spec.b}; {dt:.1f} s"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parity_sample(L, out, lay, rows=32, map="cayley", perms=None, int8=False):
    """Frobenius-relative error of sampled token rows of y and g_x against the
    oracle's materialised weight (the full-size parity tests do more)."""
    import oracle.poetx_oracle as O
    import torch
    s = L.spec
    build = O.orthogonal_blocks if map == "cayley" else O.orthogonal_blocks_cnp
    R, _ = build(L.theta_R, s.b, s.d_out)
    Pb, _ = build(L.theta_P, s.b, s.d_in)
    W0 = O.dequantize_rows(*O.quantize_rows(L.W0)) if int8 else L.W0
    if perms is None:
        W = O.materialise(W0, R, Pb, s.b, s.b)
    else:
        W = O.materialise_permuted(W0, R, Pb, s.b, s.b, perms[0], perms[1])
    idx = np.linspace(0, s.tokens - 1, rows).astype(np.int64)
    ti = torch.from_numpy(idx).cuda()
    y = out["y"][ti].float().cpu().double().numpy()
    gx = out["g_x"][ti].float().cpu().double().numpy()
    y_ref = L.x[idx] @ W.T
    gx_ref = L.g_y[idx] @ W
    return {"y_rows_fro_rel": float(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)),
            "g_x_rows_fro_rel": float(np.linalg.norm(gx - gx_ref) / np.linalg.norm(gx_ref)),
            "rows": rows}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dense_fwd_traffic.json")
# sources of the dense forward kernel (dense_kernel in dense.hip); the
# committed counter passes count only while these are unchanged
KERNEL_SOURCES = [os.path.join(ROOT, "orthogonal_equivalence_amd", "csrc", f)
                  for f in ("dense.hip", "lds_dma.h", "common.h")]


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(config):
    """L2-miss bytes per launch of the dense forward GEMM from the committed
    FETCH_SIZE / WRITE_SIZE counter passes, if they were taken on this
    workload and on the current kernel sources (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256") != sources_digest():
        return None
    if not str(t.get("workload", "")).startswith(config + ":"):
        return None
    return t.get("bytes_per_launch")


def copy_calibration(nbytes=1 << 30):
    """A plain device copy of known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters: reads nbytes and writes nbytes."""
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mlp_up_8b")
    ap.add_argument("--cpu-sample", type=int, default=8192,
                    help="tokens of the oracle's CPU-baseline sample (0 = skip)")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache steps (profiling runs)")
    ap.add_argument("--recompute-z", action="store_true",
                    help="POET-Xmem variant: the forward keeps no Z, the backward recomputes it")
    ap.add_argument("--saved-y", action="store_true",
                    help="the backward takes y in place of Z (POETX_SAVED_Y): the forward "
                         "keeps no Z")
    ap.add_argument("--permute", action="store_true",
                    help="random block-mixing permutations of R and P (W0 folded once)")
    ap.add_argument("--int8", action="store_true",
                    help="POET-XQ: the frozen weight stored as INT8 codes with per-row scales")
    ap.add_argument("--map", choices=("cayley", "cnp"), default="cayley",
                    help="orthogonal map: exact Cayley (default) or the truncated "
                         "Cayley-Neumann series")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: there is no multi-GPU path (the layer would "
              "shard over tokens, with one all-reduce of the packed generator gradients)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from orthogonal_equivalence_amd import poetx as P
    from orthogonal_equivalence_amd.inputs import CONFIGS, make_layer, make_permutations
    from orthogonal_equivalence_amd.layer import PoetxLinear, PoetxLinearSet

    specs = CONFIGS[args.config]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}

    # ---- inputs resident in HBM
    layers = []
    for s in specs:
        L = make_layer(s)
        po, pi = make_permutations(s) if args.permute else (None, None)
        lay = PoetxLinear(torch.from_numpy(L.W0).to(tdt[s.dtype]), s.b, s.b, s.dtype, device=dev,
                          recompute_z=args.recompute_z, map=args.map, perm_out=po, perm_in=pi,
                          int8=args.int8, saved_y=args.saved_y)
        lay.set_theta(torch.from_numpy(L.theta_R).float(), torch.from_numpy(L.theta_P).float())
        x = torch.from_numpy(L.x).to(tdt[s.dtype]).to(dev)
        g_y = torch.from_numpy(L.g_y).to(tdt[s.dtype]).to(dev)
        out = dict(y=torch.empty(s.tokens, s.d_out, dtype=tdt[s.dtype], device=dev),
                   z=None if args.recompute_z or args.saved_y else
                   torch.empty(s.tokens, s.d_out, dtype=tdt[s.dtype], device=dev),
                   g_x=torch.empty(s.tokens, s.d_in, dtype=tdt[s.dtype], device=dev),
                   gR=torch.empty_like(lay.theta_R), gP=torch.empty_like(lay.theta_P))
        layers.append((s, L, lay, x, g_y, out))
    # a workload of several layers with one block size rebuilds all of their
    # blocks with one call (the same work, batched), as a training step would
    layer_set = None
    if len(layers) > 1:
        try:
            layer_set = PoetxLinearSet([lay for _, _, lay, _, _, _ in layers])
        except ValueError:
            layer_set = None
    stream = torch.cuda.current_stream()
    fwd_stages = FWD_STAGES + (FWD_PERM_STAGES if args.permute else [None, None])
    bwd_stages = BWD_STAGES + (["recompute_z" if args.recompute_z else None] +
                               (BWD_PERM_STAGES if args.permute else [None, None]))
    if args.int8:
        fwd_stages += [None] * (FWD_INT8_STAGE - len(fwd_stages)) + ["int8_scale_r_fwd"]
        bwd_stages += [None] * (BWD_INT8_STAGE - len(bwd_stages)) + ["int8_scale_r_bwd"]
    while fwd_stages[-1] is None:
        fwd_stages.pop()
    while bwd_stages[-1] is None:
        bwd_stages.pop()

    def step(ev=None):
        if layer_set is not None:  # its build events are the first layer's
            e = None if ev is None else ev[0]
            if e is not None and e["build"] is not None:
                e["build"][0].record(stream)
            layer_set.build(stream)
            if e is not None and e["build"] is not None:
                e["build"][1].record(stream)
        for li, (s, _, lay, x, g_y, o) in enumerate(layers):
            e = None if ev is None else ev[li]
            if layer_set is None:
                if e is not None and e["build"] is not None:
                    e["build"][0].record(stream)
                lay.build(stream)
                if e is not None and e["build"] is not None:
                    e["build"][1].record(stream)
            lay.forward(x, o["y"], o["z"], stream=stream, events=None if e is None else e["fwd"])
            lay.backward(g_y, x, o["y"] if args.saved_y else o["z"], o["g_x"], o["gR"], o["gP"],
                         stream=stream,
                         events=None if e is None else e["bwd"])

    def make_events():
        ev = []
        for _ in layers:
            ev.append({"build": (P.Event(), P.Event()),
                       "fwd": [P.Event() for _ in range(2 * len(fwd_stages))],
                       "bwd": [P.Event() for _ in range(2 * len(bwd_stages))]})
        return ev

    def as_handles(ev):
        return [{"build": e["build"], "fwd": [x.handle for x in e["fwd"]],
                 "bwd": [x.handle for x in e["bwd"]]} for e in ev]

    # ---- the oracle on the host's cores, before any GPU timing
    cpu = None
    if args.cpu_sample > 0:
        cpu = cpu_baseline(specs[-1] if len(specs) == 1 else specs[0],
                           min(args.cpu_sample, specs[0].tokens), map=args.map,
                           permute=args.permute, int8=args.int8)

    # No garbage-collection pass from the warm-up to the end of the GPU work:
    # one in the middle of the timed steps once held the host for 36-66 ms
    # while the GPU waited for the next launch, and a collection just before
    # them leaves the GPU idle long enough for its clock to drop (the next
    # few steps then run slower), so the one collection comes first.
    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- stage breakdown: K steps with an event pair around every stage and
    # every step (slower than the timed steps by the records themselves),
    # after the W warm-up steps and before the timed ones: after the oracle's
    # seconds on the host the GPU has idled, and its clock took longer to come
    # back up than W warm-up steps (~10 ms at W = 5; the first timed steps
    # then ran 2-4 % slower than the rest), so the timed steps begin from a
    # GPU that has run the step for a while, as it would in a training loop.
    step_events = [make_events() for _ in range(args.steps)]
    handles = [as_handles(e) for e in step_events]
    per_step = [(P.Event(), P.Event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        per_step[k][0].record(stream)
        step(handles[k])
        per_step[k][1].record(stream)
    torch.cuda.synchronize()
    step_ms = [a.elapsed_ms(b) for a, b in per_step]

    # dominant kernel: the forward dense W0 GEMM (Z = U W0^T) of the largest layer
    big = max(range(len(layers)), key=lambda i: layers[i][0].d_in * layers[i][0].d_out)
    dense_stage = FWD_STAGES.index("dense_fwd")

    # ---- timed region: K steps bracketed by synchronize. Each event record
    # puts a few microseconds between two kernels, so the only ones inside are
    # one at every step boundary (per-step times, for the median) and the
    # pair around the dominant kernel's launch (its live duration).
    dense_ev = [(P.Event(), P.Event()) for _ in range(args.steps)]
    timed_handles = []
    for k in range(args.steps):
        fwd_ev = [None] * (2 * dense_stage) + [dense_ev[k][0].handle, dense_ev[k][1].handle]
        timed_handles.append([{"build": None, "fwd": fwd_ev if li == big else None, "bwd": None}
                              for li in range(len(layers))])
    bound = [P.Event() for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    bound[0].record(stream)
    for k in range(args.steps):
        step(timed_handles[k])
        bound[k + 1].record(stream)
    bound[-1].synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    total_ms = bound[0].elapsed_ms(bound[-1])
    ms_per_step = total_ms / args.steps
    timed_ms = [bound[k].elapsed_ms(bound[k + 1]) for k in range(args.steps)]
    tokens = specs[0].tokens
    value = tokens / (ms_per_step / 1e3)
    dense_ms = statistics.mean(a.elapsed_ms(b) for a, b in dense_ev)

    # ---- cold variant: K more steps, each after a 512 MB scratch write (more
    # than the 256 MB Infinity Cache), so W0 and the activations are not left
    # resident by the previous step; the write itself is outside the events
    cold_ms = []
    if not args.no_cold:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold_ev = [(P.Event(), P.Event()) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            scratch.fill_(k & 0xFF)
            cold_ev[k][0].record(stream)
            step()
            cold_ev[k][1].record(stream)
        torch.cuda.synchronize()
        cold_ms = [a.elapsed_ms(b) for a, b in cold_ev]
        del scratch
    gc.enable()


    stage_ms = {}
    if layer_set is not None:
        stage_ms["build"] = statistics.mean(
            step_events[k][0]["build"][0].elapsed_ms(step_events[k][0]["build"][1])
            for k in range(args.steps))
    for li, (s, _, _, _, _, _) in enumerate(layers):
        pre = "" if len(layers) == 1 else f"{s.name}."
        if layer_set is None:
            vals = [step_events[k][li]["build"][0].elapsed_ms(step_events[k][li]["build"][1])
                    for k in range(args.steps)]
            stage_ms[pre + "build"] = statistics.mean(vals)
        for grp, names in (("fwd", fwd_stages), ("bwd", bwd_stages)):
            for si, nm in enumerate(names):
                if nm is None:
                    continue
                vals = [step_events[k][li][grp][2 * si].elapsed_ms(step_events[k][li][grp][2 * si + 1])
                        for k in range(args.steps)]
                stage_ms[pre + nm] = statistics.mean(vals)

    sb = layers[big][0]
    dense_flops = 2.0 * sb.tokens * sb.d_in * sb.d_out
    # with bf16 and 256 x 256 R blocks the forward's R-apply runs in the dense
    # kernel's epilogue (dense_kernel<true, true, ...>), so that launch also does
    # the R-apply's 2 N d_out b flops
    fused_r = sb.dtype == "bf16" and sb.b == 256 and sb.d_out % 256 == 0
    if fused_r:
        dense_flops += 2.0 * sb.tokens * sb.d_out * sb.b
    peak = PEAK_BF16 if sb.dtype == "bf16" else PEAK_F32
    achieved = dense_flops / (dense_ms / 1e3)
    roofline = {"bound": "mfma", "achieved": achieved / 1e12, "peak": peak / 1e12, "unit": "TFLOP/s",
                "frac": achieved / peak,
                "traffic": (measured_traffic(args.config) if args.map == "cayley" and not
                            (args.permute or args.int8 or args.recompute_z or args.saved_y)
                            else None),
                "traffic_kind": "L2-miss bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a "
                                "plain copy): requests leaving the L2, answered by the Infinity "
                                "Cache or HBM; null when the kernel changed since the passes "
                                "or they were taken on another workload",
                "kernel": ("dense_fwd: Y = (U W0^T) blockdiag(R)^T, Z not written "
                           "(dense_kernel<true, true, false>" if fused_r and args.saved_y else
                           "dense_fwd: Z = U W0^T with Y = Z blockdiag(R)^T in its epilogue "
                           "(dense_kernel<true, true, true>" if fused_r else
                           "dense_fwd: Z = U W0^T (dense_kernel<true, false, true>") +
                          ": bf16, K-major W0, persistent, direct-to-LDS, 4 waves of 128x128, "
                          "16x16x32 MFMA)",
                "flops_per_launch": dense_flops, "avg_launch_ms": dense_ms}

    F = sum(layer_work(s, args.saved_y)[0] for s, *_ in layers)
    B = sum(layer_work(s, args.saved_y)[1] for s, *_ in layers)
    t_roof = max(F / PEAK_BF16, B / PEAK_HBM)
    res = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "ms_per_step_median": statistics.median(timed_ms),
        "ms_per_step_min": min(timed_ms), "ms_per_step_max": max(timed_ms),
        "ms_each_step": [round(v, 4) for v in timed_ms],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": specs[0].dtype, "data": "synthetic (seeded N(0,1) activations, N(0,1/d_in) W0, "
                                          "N(0, sigma^2) generators)",
        "config": {"workload": args.config,
                   "layers": [f"{s.name} {s.d_out}x{s.d_in} b={s.b}" for s in specs],
                   "tokens": tokens, "block": specs[0].b,
                   "variant": ("POET-Xmem (Z recomputed in the backward)" if args.recompute_z
                               else "POET-X (y kept for the backward in place of Z)"
                               if args.saved_y
                               else "POET-X (Z kept for the backward)"),
                   "orthogonal_map": ("exact Cayley" if args.map == "cayley"
                                      else "Cayley-Neumann series to Q^4"),
                   "permutations": bool(args.permute),
                   "build": ("one call for the blocks of all layers" if layer_set is not None
                             else "one call per layer"),
                   "weight": "int8 codes + per-row float32 scales" if args.int8 else specs[0].dtype},
        "roofline": roofline,
        "layer_roofline": {"flops": F, "bytes": B, "t_roof_ms": t_roof * 1e3,
                           "frac": t_roof / (ms_per_step / 1e3),
                           "tflops": F / (ms_per_step / 1e3) / 1e12},
        "wall_s": wall,
        "cold": None if not cold_ms else {
            "what": "the same step after a 512 MB scratch write (evicts the Infinity Cache); "
                    "one event pair around each step",
            "ms_per_step_median": statistics.median(cold_ms),
            "ms_per_step_mean": statistics.mean(cold_ms),
            "ms_per_step_min": min(cold_ms), "ms_per_step_max": max(cold_ms),
            "tokens_per_s_median": tokens / (statistics.median(cold_ms) / 1e3)},
        # from the instrumented steps that precede the timed ones
        "instrumented_step_ms": {"median": statistics.median(step_ms), "min": min(step_ms),
                                 "max": max(step_ms)},
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
    }
    if not args.no_parity:
        par = {}
        for s, L, lay, x, g_y, o in layers:
            par[s.name] = parity_sample(L, dict(y=o["y"], g_x=o["g_x"]), lay, map=args.map,
                                        perms=make_permutations(s) if args.permute else None,
                                        int8=args.int8)
        res["parity"] = par[specs[0].name] if len(layers) == 1 else par
    if cpu is not None:
        res["cpu_baseline"] = cpu
    res["gpu"] = torch.cuda.get_device_name(0)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
