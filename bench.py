"""Throughput of the fused encoder layer, forward + backward, on one MI355X.

Default workload: the BERT-Large layer (batch 64, sequence 128, hidden 1024,
16 heads, FFN 4096, fp16 storage / fp32 accumulation, Pre-LN, dropout 0.1)
as a stack of 24 layers with distinct layer ids.  One step = forward through
all 24 layers, then backward through all 24, every kernel in libtel.so;
inputs, weights and workspaces are resident in HBM before timing starts.

Reported: value = tokens/s of one layer's forward+backward (stack tokens/s
times the number of layers run), model TFLOP/s and its fraction of the dense
fp16 MFMA peak, per-step time percentiles, the roofline of the dominant
kernel call site (the grouped W_2 + W_1 weight-gradient launch with its
split-K reduction; timed live with HIP events around each of its launches
inside the timed steps) and of the next two call sites by time (each timed on
its own third of the layers), and the fp64 CPU oracle's throughput on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}  # MI355X dense, published
PEAK_HBM_GBS = 8000.0


def model_flops(w) -> float:
    """fwd = 2T(4H^2 + 2HF) + 4 B S^2 H; fwd+bwd = 3 x fwd (recompute not counted)."""
    T, H, F = w.batch * w.seq, w.hidden, w.ffn
    fwd = 2.0 * T * (4 * H * H + 2 * H * F) + 4.0 * w.batch * w.seq * w.seq * H
    return 3.0 * fwd


def valid_flops(w, lengths) -> float:
    """The same count over valid tokens only (token packing): projections and
    FFN on sum(len) rows, attention on len_b x len_b scores per sequence."""
    H, F = w.hidden, w.ffn
    L = [int(v) for v in lengths]
    fwd = 2.0 * sum(L) * (4 * H * H + 2 * H * F) + 4.0 * sum(v * v for v in L) * H
    return 3.0 * fwd


class Hip:
    """The few HIP runtime calls the benchmark needs for events."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self) -> int:
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    def destroy(self, e):
        self.h.hipEventDestroy(ctypes.c_void_p(e))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, n_seq: int):
    """Oracle forward + backward of n_seq sequences of the workload (fp64, host
    cores): one call that runs the forward and then the backward."""
    import oracle
    from transformer_encoder_layer_amd import synthetic as syn
    sub = w.with_(batch=n_seq)
    p = syn.layer_params(w, 0)
    x = syn.layer_input(w)[: n_seq * w.seq]
    dy = syn.upstream_grad(w)[: n_seq * w.seq]
    lengths = syn.seq_lengths(w)[:n_seq]
    cfg = oracle.LayerCfg(n_seq, w.seq, w.hidden, w.heads, w.ffn, pre_ln=w.pre_ln, training=True,
                          attn_p=float(np.float32(w.attn_p)), hidden_p=float(np.float32(w.hidden_p)),
                          seed=w.seed, step=0, layer_id=0)
    threads = oracle.omp_threads()
    t0 = time.perf_counter()
    oracle.layer_backward(cfg, p, x, lengths, dy, ln_invertible=w.normalize_invertible, want_y=True)
    dt = time.perf_counter() - t0
    return {"value": n_seq * w.seq / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_seq} of {w.batch} sequences ({n_seq * w.seq} tokens), one layer forward+backward, "
                      f"fp64, {dt:.2f} s", "seconds": dt,
            "model_gflops": model_flops(sub) / dt / 1e9, "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)), "omp_threads": threads}


COPY_BYTES = 1 << 30


def copy_calibration(torch):
    """Five device-to-device copies of 1 GiB: under a counter run, FETCH_SIZE and
    WRITE_SIZE of each copy dispatch should read 1 GiB; the ratio scales the
    counters read for the layer's kernels to bytes."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 5}))


def kernel_sources_digest() -> str:
    """sha256 over the GEMM sources: stored counter readings are only valid for them."""
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "gemm.h", "mfma_common.h", "tel_common.h", "fastdiv.h"):
        with open(os.path.join(ROOT, "transformer_encoder_layer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE on
# the BERT-Large layer, scaled by the copy calibration; keyed by the digest of
# the kernel sources they were taken on (a changed kernel reports null).
MEASURED_TRAFFIC = {
    # W2 + W1 weight-gradient pair: the grouped GEMM launch (its split-K reduce launch, 84.0 MB, apart)
    ("ffn_wgrad_pair", "bert_large"): ("58f015700fac927a", 268722874),
    # W_o + W_qkv pair: the grouped GEMM launch (its reduce with the LayerNorm gamma/beta sums, 109.2 MB, apart)
    ("attn_wgrad_pair", "bert_large"): ("58f015700fac927a", 197445846),
    # FFN1 forward (GELU epilogue)
    ("ffn1_fwd", "bert_large"): ("58f015700fac927a", 235330518),
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="bert_large")
    ap.add_argument("--layers", type=int, default=0, help="override the stack depth")
    ap.add_argument("--kernel", default="ffn_wgrad_pair", help="call site whose roofline is reported")
    ap.add_argument("--also", default="ffn_wgrad_reduce,ffn1_fwd,attn_wgrad_pair",
                    help="further call sites timed (comma-separated), each on its own share of the layers")
    ap.add_argument("--cpu-seqs", type=int, default=64, help="sequences in the oracle sample (BERT-Large: the whole batch, about 10 s on 16 host threads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stochastic", action="store_true",
                    help="relaxed-determinism mode (the weight-gradient pairs add their k-splits atomically)")
    ap.add_argument("--pack", action="store_true",
                    help="token packing: run the layers on the valid tokens of a padded workload")
    ap.add_argument("--unchained", action="store_true",
                    help="Pre-LN stacks: each layer applies its own site-2 dropout to dy, instead of the layer "
                         "above doing it in its LayerNorm-1 backward")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain device copies of 1 GiB (scale for the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(data-parallel sharding of the layer is designed, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    from transformer_encoder_layer_amd import binding as B
    from transformer_encoder_layer_amd import synthetic as syn
    from transformer_encoder_layer_amd.layer import LayerConfig, pld_gates

    w = syn.WORKLOADS[args.workload]
    n_layers = args.layers or w.layers
    dev = torch.device("cuda:0")
    dt = syn.torch_dtype(w.dtype)
    T, H = w.tokens, w.hidden
    pack = bool(args.pack and w.lengths is not None)
    valid = int(syn.seq_lengths(w).sum()) if w.lengths is not None else T

    # ---- layers (distinct ids, weights from the seeded generator)
    handles, params, grads, saved = [], [], [], []
    for l in range(n_layers):
        cfg = LayerConfig(w.batch, w.seq, w.hidden, w.heads, w.ffn, float(np.float32(w.attn_p)),
                          float(np.float32(w.hidden_p)), w.pre_ln, w.seed, l, dt, 1e-12,
                          w.attn_dropout_checkpoint, w.normalize_invertible, w.gelu_checkpoint, pack_tokens=pack,
                          stochastic_mode=args.stochastic)
        h = B.tel_layer_create(cfg.to_c())
        if pack:
            B.tel_layer_set_valid_tokens(h, valid)
        handles.append(h)
        p64 = syn.layer_params(w, l)
        P = {n: syn.to_storage(p64[n], w.dtype).to(dev) for n in B.PARAM_NAMES}
        params.append(P)
        grads.append({n: torch.empty_like(P[n]) for n in B.PARAM_NAMES})
        sv, sc = B.tel_layer_workspace_bytes(h)
        saved.append(torch.empty(sv, dtype=torch.uint8, device=dev))
    scratch = torch.empty(max(B.tel_layer_workspace_bytes(h)[1] for h in handles), dtype=torch.uint8,
                          device=dev)
    cparams = [B.make_params(P) for P in params]
    cgrads = [B.make_grads(G) for G in grads]
    x0 = syn.to_storage(syn.layer_input(w), w.dtype).to(dev)
    dy_top = syn.to_storage(syn.upstream_grad(w), w.dtype).to(dev)
    lengths = torch.from_numpy(syn.seq_lengths(w)).to(dev) if w.lengths is not None else None
    acts = [x0] + [torch.empty_like(x0) for _ in range(n_layers)]
    dgrads = [torch.empty_like(x0) for _ in range(n_layers)] + [dy_top]

    # progressive layer dropping: gates of this step (memory-saving stack)
    step_id = w.pld[2] if w.pld else 0
    if w.pld:
        theta = B.tel_pld_theta(step_id, w.pld[0], w.pld[1])
        gates = pld_gates(w.seed, n_layers, step_id, w.pld[0], w.pld[1])
    else:
        theta, gates = 1.0, [True] * n_layers
    run = [l for l in range(n_layers) if gates[l]]
    stream = torch.cuda.current_stream().cuda_stream
    # Pre-LN stacks chain the backward: each layer's LayerNorm-1 backward also
    # writes the next run layer's site-2 masked gradient (two buffers in turn)
    chain = w.pre_ln and not pack and not args.unchained
    dxd = [torch.empty_like(x0), torch.empty_like(x0)] if chain else None

    def step():
        # skipped layers are the identity: their input buffer is passed on unchanged
        cur = x0
        inputs = {}
        for l in run:
            inputs[l] = cur
            B.tel_layer_forward(handles[l], cparams[l], cur, lengths, 1, step_id, acts[l + 1], saved[l], scratch,
                                stream)
            cur = acts[l + 1]
        g, gd = dy_top, None
        order = run[::-1]
        for i, l in enumerate(order):
            if chain:
                below = handles[order[i + 1]] if i + 1 < len(order) else None
                out_d = dxd[i % 2] if below is not None else None
                B.tel_layer_backward_chain(handles[l], cparams[l], inputs[l], lengths, 1, step_id, g, gd, saved[l],
                                           scratch, dgrads[l], below, out_d, cgrads[l], stream)
                gd = out_d
            else:
                B.tel_layer_backward(handles[l], cparams[l], inputs[l], lengths, 1, step_id, g, saved[l], scratch,
                                     dgrads[l], cgrads[l], stream)
            g = dgrads[l]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # live per-kernel timing during the timed steps: the roofline call site on
    # every layer when it is the only one, else each timed call site on its
    # own share of the layers (every layer has the same shapes)
    hip = Hip()
    sites = [args.kernel] + [k for k in args.also.split(",") if k and k != args.kernel]
    site_of = {l: sites[i * len(sites) // len(run)] for i, l in enumerate(run)}
    ev = {l: ([hip.event() for _ in range(args.steps)], [hip.event() for _ in range(args.steps)]) for l in run}
    keep_alive = [B.tel_debug_kernel_events(handles[l], B.KERNELS[site_of[l]], ev[l][0], ev[l][1]) for l in run]
    t_start, t_stop = hip.event(), hip.event()
    step_ev = [hip.event() for _ in range(args.steps + 1)]

    torch.cuda.synchronize()
    hip.h.hipEventRecord(ctypes.c_void_p(t_start), ctypes.c_void_p(stream))
    t0 = time.perf_counter()
    for i in range(args.steps):
        hip.h.hipEventRecord(ctypes.c_void_p(step_ev[i]), ctypes.c_void_p(stream))
        step()
    hip.h.hipEventRecord(ctypes.c_void_p(step_ev[-1]), ctypes.c_void_p(stream))
    hip.h.hipEventRecord(ctypes.c_void_p(t_stop), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = hip.elapsed_ms(t_start, t_stop)
    step_ms = np.array([hip.elapsed_ms(step_ev[i], step_ev[i + 1]) for i in range(args.steps)])
    for l in run:
        B.tel_debug_kernel_events(handles[l], -1, None, None)
    del keep_alive
    site_ms = {k: [] for k in sites}
    for l in run:
        for a, b in zip(*ev[l]):
            site_ms[site_of[l]].append(hip.elapsed_ms(a, b))

    ms_per_step = total_ms / args.steps
    n_run = len(run)
    layer_tokens_per_s = T * n_run / (ms_per_step / 1e3)
    flops = valid_flops(w, syn.seq_lengths(w)) if pack else model_flops(w)
    tflops = flops * n_run / (ms_per_step / 1e3) / 1e12
    peak = PEAK_MFMA_TFLOPS[w.dtype]

    # roofline of each timed call site (algorithmic work per launch)
    F = w.ffn
    Tg = (valid + 255) // 256 * 256 if pack else T  # rows the GEMMs and LayerNorms run on
    gemm_flops = {"qkv_fwd": 2.0 * Tg * H * 3 * H, "out_fwd": 2.0 * Tg * H * H, "ffn1_fwd": 2.0 * Tg * H * F,
                  "ffn2_fwd": 2.0 * Tg * F * H, "ffn2_dgrad": 2.0 * Tg * H * F, "ffn2_wgrad": 2.0 * Tg * H * F,
                  "ffn1_dgrad": 2.0 * Tg * F * H, "ffn1_wgrad": 2.0 * Tg * F * H, "out_dgrad": 2.0 * Tg * H * H,
                  "out_wgrad": 2.0 * Tg * H * H, "qkv_dgrad": 2.0 * Tg * 3 * H * H, "qkv_wgrad": 2.0 * Tg * 3 * H * H,
                  "ffn_wgrad_pair": 4.0 * Tg * H * F, "attn_wgrad_pair": 2.0 * Tg * H * H + 2.0 * Tg * 3 * H * H}
    digest = kernel_sources_digest()

    def roofline(site):
        ms = site_ms[site]
        if not ms:
            return {"kernel": site, "launches": 0}
        avg_ms = float(np.mean(ms))
        if site.endswith("_wgrad_reduce"):  # the launch after a pair: its time, and the pair's rate with it
            pair = site.replace("_reduce", "_pair")
            out_r = {"kernel": site, "avg_launch_us": round(avg_ms * 1e3, 2), "launches": len(ms)}
            if site_ms.get(pair):
                both = float(np.mean(site_ms[pair])) + avg_ms
                ach = gemm_flops[pair] / (both / 1e3) / 1e12
                out_r["pair_with_reduce"] = {"achieved": round(ach, 1), "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                                             "avg_us": round(both * 1e3, 2)}
            return out_r
        if site in gemm_flops:
            ach = gemm_flops[site] / (avg_ms / 1e3) / 1e12
            meas = MEASURED_TRAFFIC.get((site, w.name))
            traffic = meas[1] if meas and meas[0] == digest and not pack else None
            out_s = {"kernel": site, "bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(ach / peak, 4), "traffic": traffic, "avg_launch_us": round(avg_ms * 1e3, 2),
                     "launches": len(ms), "algorithmic_per_launch": gemm_flops[site]}
            if site.endswith("_wgrad_pair"):  # a grouped launch always runs the four-wave 256x256 kernel
                out_s["symbol"] = f"gemm_dl4_kernel<{w.dtype},256,256,0,0,0>"
            return out_s
        e = 2 if w.dtype != "f32" else 4
        ln_bytes = {"ln1_fwd": 2 * Tg * H * e + 8 * Tg, "ln2_fwd": Tg * H * (4 + e) + 8 * Tg}
        byts = ln_bytes.get(site, float("nan"))
        ach = byts / (avg_ms / 1e3) / 1e9
        return {"kernel": site, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None,
                "avg_launch_us": round(avg_ms * 1e3, 2), "launches": len(ms), "algorithmic_per_launch": byts}

    roof = roofline(sites[0])
    others = [roofline(k) for k in sites[1:]]
    for o in others:  # the dominant pair's rate including the launch after it
        if o.get("kernel") == sites[0].replace("_pair", "_reduce") and "pair_with_reduce" in o:
            roof["with_reduce"] = dict(o["pair_with_reduce"], reduce_avg_us=o["avg_launch_us"])
    shape = (f"{'BERT-Large' if w.name == 'bert_large' else w.name} layer B{w.batch} S{w.seq} H{w.hidden} "
             f"{ {'f16': 'fp16', 'bf16': 'bf16', 'f32': 'fp32'}[w.dtype]}{', token packing' if pack else ''}")

    out = {
        "metric": f"fwd+bwd tokens/sec and TFLOP/s (% MFMA peak), {shape}",
        "value": round(layer_tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: batch {w.batch}, seq {w.seq}, hidden {w.hidden}, heads {w.heads}, "
                               f"ffn {w.ffn}, {'Pre' if w.pre_ln else 'Post'}-LN, {w.dtype}, dropout "
                               f"{w.attn_p}/{w.hidden_p}, {n_layers}-layer stack"
                               + (f", PLD theta={theta:.5f} keeps {n_run}" if w.pld else "")
                               + (f", token packing ({valid} valid of {T} tokens)" if pack else "")
                               + (", stochastic mode" if args.stochastic else ""),
                   "batch": w.batch, "seq_len": w.seq, "hidden": w.hidden, "heads": w.heads, "ffn": w.ffn,
                   "layers": n_layers, "layers_run": n_run, "parallelism": "single GPU"},
        "tflops": round(tflops, 1),
        "pct_mfma_peak": round(100 * tflops / peak, 2),
        "stack_tokens_per_s": round(T / (ms_per_step / 1e3), 1),
        "ms_per_layer_fwd_bwd": round(ms_per_step / n_run, 4),
        "valid_tokens_per_s": round(valid * n_run / (ms_per_step / 1e3), 1),
        "token_packing": pack,
        "chained_backward": chain,
        "wall_s_timed": round(wall, 3),
        "step_ms": {"median": round(float(np.median(step_ms)), 4), "p10": round(float(np.percentile(step_ms, 10)), 4),
                    "p90": round(float(np.percentile(step_ms, 90)), 4)},
        "roofline": roof,
        "kernels": [roof] + others,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, min(args.cpu_seqs, w.batch))
    for e in [t_start, t_stop] + step_ev + [x for l in run for x in ev[l][0] + ev[l][1]]:
        hip.destroy(e)
    for h in handles:
        B.tel_layer_destroy(h)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
