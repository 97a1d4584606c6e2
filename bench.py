#!/usr/bin/env python
"""Aggregate decode throughput of decode_step_batch on one MI355X.

Workload (synthetic, seeded): a Llama-3-8B-shaped random-init decoder in bf16
(32 layers, d_model 4096, 32/8 heads of 128, SwiGLU 14336, vocab 128256,
RoPE theta 500000), B = 8 live sequences whose contexts are uniform in
[512, 4096] (K/V histories drawn by ``synth`` and appended to the slabs),
greedy decoding with the next tokens kept on the device. A step is one
``decode_step_batch`` over all B rows: embed, 32 layers (norm, QKV, RoPE +
append, ragged attention, O + residual, norm, gate/up + SwiGLU, down +
residual), final norm, lm_head, argmax.

Prints ONE JSON line on stdout (progress goes to stderr):
- value: aggregate tok/s = B * steps / timed seconds (inputs resident in HBM)
- roofline: the dominant kernel (the weight-streaming product with the fused
  SwiGLU epilogue) timed with HIP events on its own launch stream over the
  timed region, against the 8 TB/s HBM peak
- cpu_baseline: the CPU oracle timed on one decode step of the same rows
- sweep: tok/s at B = 1..64 on the same model (scaling check)

Other workloads (``--workload``), each printing its own JSON line:
- mistral7b-int4: Mistral-7B-shaped model with 4-bit affine weights (group 64),
  B = 8 (sweep 1, 4, 8, 16), contexts uniform in [1024, 8192]; roofline on the
  fused-dequant gate/up product.
- llama8b-long: the 8B-shape bf16 model with B = 8 rows at 32768-token contexts,
  128 steps; roofline on decode attention (the K/V stream dominates the step).
- llama8b-long-kv8: the same with affine 8-bit K/V slabs (codes + float32 scale and bias per
  64 dims): the K/V stream shrinks to 144 of 256 bytes per token, layer and KV head.
- llama8b-long-kv4: the same with 4-bit codes (80 bytes per token, layer and KV head).
- continuous: the 8B-shape bf16 model under continuous batching with the batch cap
  swept over 1..64: Poisson arrivals (in decode ticks, offered concurrency about
  1.25 x cap), prompts uniform in [256, 2048] sharing a 1024-token prefix,
  generation lengths uniform in [64, 512]. Joiners are admitted between steps
  with one segmented prefill, rows retire when their length is reached.
- prefill: prefill_segmented of K = 16 prompts with lengths uniform in
  [64, 1024] (7797 tokens) on the 8B-shape bf16 model into fresh slabs; value in
  prefill tok/s; roofline on the dense gate/up + SwiGLU product against the bf16
  MFMA peak (algorithmic 2*T*N*K flop; the hi/lo activation pairs run twice that
  on the matrix cores).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "aggregate decode tok/s at B=1..64, 8B-shape bf16; achieved HBM GB/s"
WORKLOADS = {
    "llama8b-b8": {"shape": "llama3-8b-shape", "steps": 256, "batch": 8, "sweep": "1,2,4,8,16,32,64", "ctx_lo": 512,
                   "ctx_hi": 4096, "roofline": "gate_up", "hist_seed": 1},
    "mistral7b-int4": {"shape": "mistral7b-shape-int4", "steps": 128, "batch": 8, "sweep": "1,4,8,16",
                       "ctx_lo": 1024, "ctx_hi": 8192, "roofline": "gate_up", "hist_seed": 4},
    "llama8b-long": {"shape": "llama3-8b-shape", "steps": 128, "batch": 8, "sweep": "", "ctx_lo": 32768,
                     "ctx_hi": 32768, "roofline": "attention", "hist_seed": 5},
    "llama8b-long-kv8": {"shape": "llama3-8b-shape", "steps": 128, "batch": 8, "sweep": "", "ctx_lo": 32768,
                         "ctx_hi": 32768, "roofline": "attention", "hist_seed": 5, "kv_format": "affine8"},
    "llama8b-long-kv4": {"shape": "llama3-8b-shape", "steps": 128, "batch": 8, "sweep": "", "ctx_lo": 32768,
                         "ctx_hi": 32768, "roofline": "attention", "hist_seed": 5, "kv_format": "affine4"},
    "continuous": {"shape": "llama3-8b-shape", "steps": 0, "batch": 64, "sweep": "1,2,4,8,16,32,64", "ctx_lo": 256,
                   "ctx_hi": 2048, "roofline": "gate_up", "hist_seed": 2},
    "prefill": {"shape": "llama3-8b-shape", "steps": 8, "batch": 16, "sweep": "", "ctx_lo": 64, "ctx_hi": 1024,
                "roofline": "gate_up", "hist_seed": 5},
}
MFMA_PEAK_TFLOPS_BF16 = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gate_up_llama8b_b8.md")
KERNEL_SRC = os.path.join(ROOT, "continuous_batching_decode_amd", "csrc", "gemm_skinny.hip")


def log(*a):
    print("[bench %6.1fs]" % (time.time() - T0), *a, file=sys.stderr, flush=True)


T0 = time.time()


# per workload: the committed counter summary of its roofline kernel and that kernel's source file
ATTN_SRC = os.path.join(ROOT, "continuous_batching_decode_amd", "csrc", "attention.hip")
COMMITTED = {
    "llama8b-b8": (TRAFFIC_FILE, KERNEL_SRC),
    "mistral7b-int4": (os.path.join(ROOT, "profiles", "traffic_gate_up_int4_mistral7b_b8.md"), KERNEL_SRC),
    "llama8b-long": (os.path.join(ROOT, "profiles", "traffic_attention_llama8b_long.md"), ATTN_SRC),
    "llama8b-long-kv8": (os.path.join(ROOT, "profiles", "traffic_attention_q8_llama8b_long.md"), ATTN_SRC),
}


def source_hash(path=KERNEL_SRC) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def committed_profile(field, workload="llama8b-b8"):
    """A figure of the workload's roofline kernel from its committed profile summary (HBM bytes per
    launch from the counters, or its average duration in the kernel trace), or None when absent or
    taken on a different kernel source."""
    if workload not in COMMITTED or not os.path.exists(COMMITTED[workload][0]):
        return None
    summary, src = COMMITTED[workload]
    text = open(summary).read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(field + r":\s*([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != source_hash(src):
        return None
    return float(t.group(1))


def committed_traffic(workload="llama8b-b8"):
    return committed_profile("traffic_bytes_per_launch", workload)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--sweep", default=None, help="batch sizes for the scaling sweep ('' = none)")
    ap.add_argument("--sweep-steps", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--roofline-every", type=int, default=31,
                    help="time one roofline-kernel launch in this many inside the timed region")
    ap.add_argument("--ctx-lo", type=int, default=None)
    ap.add_argument("--ctx-hi", type=int, default=None)
    ap.add_argument("--workload", default="llama8b-b8", choices=sorted(WORKLOADS))
    ap.add_argument("--prefill-chunk", type=int, default=2048,
                    help="continuous workload: prefill tokens per tick (joiner prompts continue over ticks); "
                         "0 = whole prompts per call")
    ap.add_argument("--share-prefix", type=int, default=1, choices=[0, 1],
                    help="continuous workload: joiners fork the prompts' common 1024-token prefix from one "
                         "prefilled holder sequence (kvslab_fork) and prefill only the rest; 0 = whole prompts")
    ap.add_argument("--parity-rows", type=int, default=0,
                    help="decode workloads: run the oracle (parity and cpu baseline) on the first this many rows "
                         "only (0 = all rows; long-context workloads run it only when this is set)")
    ap.add_argument("--fill", default="seeded", choices=["seeded", "copy"],
                    help="decode workloads: 'copy' draws row 0's K/V history and copies it on the device to the "
                         "other rows (the same bytes streamed, less host time for 32k-token histories)")
    ap.add_argument("--no-extras", action="store_true",
                    help="default workload: skip the compact int4, prefill and 32k-context sub-benchmarks")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only copy a device buffer of this many MiB 5 times (a plain copy of known size, "
                         "used to calibrate HBM byte counters), then exit")
    args = ap.parse_args()
    wl = WORKLOADS[args.workload]
    for k in ("steps", "batch", "sweep", "ctx_lo", "ctx_hi"):
        if getattr(args, k) is None:
            setattr(args, k, wl[k])
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (data parallel: each GPU "
              "would run its own independent engine over its own sequences). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import continuous_batching_decode_amd as cbd
    import synth

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        rates = {}
        for name, op in (("copy", lambda: dst.copy_(src)),  # device-to-device copy: n bytes read, n written
                         ("elementwise", lambda: torch.bitwise_not(src, out=dst))):  # the same traffic
            op()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                op()
            e1.record()
            torch.cuda.synchronize()
            rates[name] = round(2 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        log("copy probe: 2 x 5 passes over %d MiB: %s GB/s (bytes read + written)" % (args.copy_probe_mib, rates))
        print(json.dumps({"copy_probe_mib": args.copy_probe_mib, "GBps_read_plus_written": rates}), flush=True)
        return

    if args.workload == "continuous":
        return run_continuous(args, wl, torch, cbd, synth)
    if args.workload == "prefill":
        return run_prefill(args, wl, torch, cbd, synth)
    shape = synth.SHAPES[wl["shape"]]
    B = args.batch
    sweep = [int(x) for x in args.sweep.split(",") if x.strip()]
    n_rows = max([B] + sweep)
    ctx = synth.uniform_lengths(wl["hist_seed"], B, args.ctx_lo, args.ctx_hi).astype(int)
    ctx_main = ctx.copy()
    # sweep-only rows (beyond B) reuse the main rows' histories
    ctx = np.array([ctx[r % B] for r in range(n_rows)], dtype=int)
    grow = args.warmup + args.steps + 1 + (0 if args.no_breakdown else min(16, args.steps)) + \
           len(sweep) * (args.sweep_steps + 4)
    caps = [int(c) + grow + 8 for c in ctx]
    gran = 256
    arena_tokens = sum((c + gran - 1) // gran * gran for c in caps)
    kv_format = wl.get("kv_format", "bf16")
    kv_tok = cbd.kv_bytes_per_token(shape, kv_format)
    max_pos = int(max(caps)) + gran

    w_bytes = shape.streamed_params() * (2 if shape.weight_format == "bf16" else 0.5625)
    log("%s: generating %s weights (%.2f GB streamed per step)" % (args.workload, shape.name, w_bytes / 1e9))
    weights = synth.make_weights(shape, seed=0)
    log("uploading weights; arena %.1f GB" % (arena_tokens * kv_tok / 1e9))
    eng = cbd.Engine(weights, arena_bytes=arena_tokens * kv_tok, max_batch=64, max_prefill_tokens=64,
                     max_position=max_pos, kv_format=kv_format)
    dev = torch.device("cuda:0")
    ids = [eng.alloc(c) for c in caps]
    hist = []
    long_ctx = args.workload.startswith("llama8b-long")
    oracle_rows = B if args.parity_rows <= 0 else min(B, args.parity_rows)
    run_oracle = not args.no_cpu_baseline and (not long_ctx or args.parity_rows > 0)
    drawn = B if args.fill == "seeded" else 1  # rows whose history is drawn on the host
    for r in range(drawn):
        keep = run_oracle and r < oracle_rows  # the oracle needs these histories
        # seeded K/V, appended in chunks of tokens (the same values as synth.kv_history of the whole row)
        n = int(ctx[r])
        std = shape.weight_std * float(np.sqrt(shape.d_model))
        per_layer = n * shape.kv_dim
        ks, vs = [], []
        for t0 in range(0, n, 4096):
            cn = min(4096, n - t0)
            kc = np.stack([synth.normal_bf16(wl["hist_seed"], 10_000_000 + 2 * r, (cn, shape.n_kv_heads, shape.head_dim),
                                             std, offset=l * per_layer + t0 * shape.kv_dim) for l in range(shape.n_layers)])
            vc = np.stack([synth.normal_bf16(wl["hist_seed"], 10_000_001 + 2 * r, (cn, shape.n_kv_heads, shape.head_dim),
                                             std, offset=l * per_layer + t0 * shape.kv_dim) for l in range(shape.n_layers)])
            eng.append(ids[r], torch.from_numpy(kc.view(np.int16)).to(dev), torch.from_numpy(vc.view(np.int16)).to(dev))
            if keep:
                ks.append(kc)
                vs.append(vc)
        if keep:
            hist.append((np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)))
    if (n_rows > B or drawn < B) and kv_format != "bf16":
        raise SystemExit("rows filled by device copies of bf16 slabs; not available with %s K/V" % kv_format)
    for r in range(drawn, n_rows):
        # rows not drawn on the host (sweep-only rows; with --fill copy every row past 0) copy the history
        # of a drawn row on the device
        src = r % B if r >= B else 0
        k, v = eng.read(ids[src], 0, min(int(ctx[src]), int(ctx[r])))
        eng.append(ids[r], k, v)
        if drawn < B and r < B and int(ctx[r]) > int(ctx[src]):
            raise SystemExit("--fill copy needs rows no longer than row 0")
        del k, v
    torch.cuda.synchronize()
    log("slabs ready: contexts %s" % list(ctx_main))

    V = shape.vocab
    first_tok = synth.prompts(2, [n_rows], V)[0].astype(np.int32)
    logits = torch.empty((64, V), dtype=torch.float32, device=dev)
    tok_a = torch.from_numpy(first_tok).to(dev)
    tok_b = torch.empty(64, dtype=torch.int32, device=dev)
    main_ids = ids[:B]

    # step 0 (first warmup step) doubles as a parity sample against the oracle below
    eng.decode_step_batch(main_ids, tok_a[:B], logits[:B], tok_b[:B])
    torch.cuda.synchronize()
    first_logits = logits[:B].cpu().numpy().astype(np.float64)
    tok_a, tok_b = tok_b, tok_a
    for _ in range(max(0, args.warmup - 1)):
        eng.decode_step_batch(main_ids, tok_a[:B], logits[:B], tok_b[:B])
        tok_a, tok_b = tok_b, tok_a
    torch.cuda.synchronize()

    log("timing %d steps at B=%d" % (args.steps, B))
    rk = wl["roofline"]
    # one launch in `every` of the roofline kernel carries timing events (each costs the stream a few
    # microseconds); a stride co-prime to the layer count cycles the sample through the layers
    eng.profile_begin([rk], max_launches=shape.n_layers * args.steps + 64, every=args.roofline_every)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        eng.decode_step_batch(main_ids, tok_a[:B], logits[:B], tok_b[:B])
        tok_a, tok_b = tok_b, tok_a
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = eng.profile_end()
    secs = t1 - t0
    ms_step = secs * 1e3 / args.steps
    tokps = B * args.steps / secs

    # algorithmic bytes per step, averaged over the timed steps
    mean_t = float(np.mean(ctx_main)) + args.warmup + (args.steps - 1) / 2.0
    step_bytes = w_bytes + B * (mean_t + 1) * kv_tok + B * kv_tok + B * V * 4
    step_gbps = step_bytes / (ms_step * 1e-3) / 1e9

    gu = prof[rk]
    per_launch_bytes = gu["bytes"] / gu["launches"]
    avg_ms = gu["total_ms"] / gu["launches"]
    achieved = per_launch_bytes / (avg_ms * 1e-3) / 1e9
    kernel_desc = {
        "gate_up": "ksplit_gemm_kernel: gate/up weight stream with fused SwiGLU (%s weights), %s, B=%d" % (
            shape.weight_format, shape.name, B),
        "attention": "%s: RoPE + K/V append + ragged GQA attention, %s K/V, %s, B=%d at %d-token contexts" % (
            "decode_attention_q8_kernel" if kv_format != "bf16" else "decode_attention_kernel", kv_format,
            shape.name, B, args.ctx_lo),
    }[rk]
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": committed_traffic(args.workload),
                "kernel": kernel_desc, "bytes_per_launch": per_launch_bytes, "avg_launch_us": round(avg_ms * 1e3, 2),
                "launches": gu["launches"],
                "kernel_source_sha256_16": source_hash(COMMITTED.get(args.workload, (None, KERNEL_SRC))[1])}
    if args.workload in COMMITTED:
        # the same kernel's average in the committed rocprofv3 trace of this command: the live events
        # run a few microseconds longer on the launches they bracket (their completion signalling)
        tr = committed_profile("kernel_trace_avg_us", args.workload)
        if tr:
            roofline["trace_avg_launch_us"] = tr
            roofline["frac_at_trace_avg"] = round(per_launch_bytes / (tr * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
    log("B=%d: %.1f tok/s, %.3f ms/step, step %.0f GB/s; %s %.1f us -> %.0f GB/s" % (
        B, tokps, ms_step, step_gbps, rk, avg_ms * 1e3, achieved))

    breakdown = None
    if not args.no_breakdown:
        nb = min(16, args.steps)
        eng.profile_begin(cbd.KERNEL_KINDS, max_launches=nb * (shape.n_layers * 10 + 8))
        for _ in range(nb):
            eng.decode_step_batch(main_ids, tok_a[:B], logits[:B], tok_b[:B])
            tok_a, tok_b = tok_b, tok_a
        torch.cuda.synchronize()
        p = eng.profile_end()
        breakdown = {k: {"ms_per_step": round(v["total_ms"] / nb, 4),
                         "GBps": round(v["bytes"] / (v["total_ms"] * 1e-3) / 1e9, 1) if v["total_ms"] else None,
                         "launches_per_step": v["launches"] // nb} for k, v in p.items()}
        log("breakdown (event-timed, %d steps): %s" % (nb, json.dumps(breakdown)))

    # seeded top-p sampling of the step's logits rows (temperature 0.8, top_p 0.95), beside greedy argmax
    sampling = None
    if not args.no_breakdown:
        s_t, s_p, s_seed = [0.8] * B, [0.95] * B, list(range(1, B + 1))
        s_out = torch.empty(B, dtype=torch.int32, device=dev)
        g_out = torch.empty(B, dtype=torch.int32, device=dev)
        for _ in range(3):
            eng.sample_top_p(logits[:B], s_t, s_p, s_seed, [0] * B, s_out)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        for i in range(50):
            eng.sample_top_p(logits[:B], s_t, s_p, s_seed, [i] * B, s_out)
        ev[1].record()
        for i in range(50):
            eng.greedy_argmax(logits[:B], g_out)
        ev[2].record()
        torch.cuda.synchronize()
        samp_logits = logits[:B].cpu().numpy().astype(np.float64)
        sampling = {"rows": B, "vocab": V, "temperature": 0.8, "top_p": 0.95,
                    "sample_us_per_call": round(ev[0].elapsed_time(ev[1]) * 1e3 / 50, 2),
                    "argmax_us_per_call": round(ev[1].elapsed_time(ev[2]) * 1e3 / 50, 2),
                    "sample_index": 49, "tokens": [int(x) for x in s_out.cpu().numpy()]}
        log("sampling: %s" % json.dumps({k: v for k, v in sampling.items() if k != "tokens"}))

    sweep_out = {}
    for b in sweep:
        sids = ids[:b]
        for _ in range(4):
            eng.decode_step_batch(sids, tok_a[:b], logits[:b], tok_b[:b])
            tok_a, tok_b = tok_b, tok_a
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        for _ in range(args.sweep_steps):
            eng.decode_step_batch(sids, tok_a[:b], logits[:b], tok_b[:b])
            tok_a, tok_b = tok_b, tok_a
        torch.cuda.synchronize()
        s = time.perf_counter() - s0
        ms = s * 1e3 / args.sweep_steps
        lens = np.array([eng.length(i) for i in sids], dtype=np.float64) - args.sweep_steps / 2.0
        by = w_bytes + float(np.sum(lens + 1)) * kv_tok + b * kv_tok + b * V * 4
        sweep_out[str(b)] = {"tok_s": round(b * args.sweep_steps / s, 1), "ms_per_step": round(ms, 4),
                             "GBps": round(by / (ms * 1e-3) / 1e9, 1)}
        log("sweep B=%d: %s" % (b, sweep_out[str(b)]))

    cpu = None
    parity = None
    if run_oracle:
        from oracle import OracleModel, greedy
        cores, blas = host_cores()
        R = oracle_rows
        log("cpu baseline: oracle, one decode step of %d of the %d rows (host cores %d, BLAS threads %d)" % (
            R, B, cores, blas))
        orc = OracleModel(weights)
        oids = []
        for r in range(R):
            o = orc.new_sequence()
            orc.append_history(o, hist[r][0], hist[r][1])
            oids.append(o)
        hist = None
        c0 = time.perf_counter()
        ref = orc.decode_step_batch(oids, first_tok[:R].astype(np.int64))
        csecs = time.perf_counter() - c0
        cpu = {"value": round(R / csecs, 4), "unit": "tok/s", "cores": int(cores), "blas_threads": int(blas),
               "kind": "oracle",
               "sample": "one decode_step_batch of %d of the %d rows at their seeded contexts (float64, all %d "
                         "layers + lm_head), %.1f s" % (R, B, shape.n_layers, csecs)}
        errs = np.max(np.abs(first_logits[:R] - ref), axis=1) / np.max(np.abs(ref), axis=1)
        parity = {"max_rel_err": float(np.max(errs)), "tol": 1e-2,
                  "greedy_match": int(np.sum(greedy(first_logits[:R]) == greedy(ref))), "rows": R}
        log("cpu baseline %.2f s/step; parity %s" % (csecs, parity))
        if sampling is not None:
            # the sampled tokens against the oracle's selection on the same (GPU) logits rows
            from oracle import sample_rows
            want = sample_rows(samp_logits, [0.8] * B, [0.95] * B, list(range(1, B + 1)), [49] * B)
            sampling["oracle_match"] = int(np.sum(want == np.array(sampling["tokens"])))

    out = {"metric": METRIC, "value": round(tokps, 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16" if shape.weight_format == "bf16" else "int4-affine/bf16",
           "data": "synthetic" if args.fill == "seeded" else
                   "synthetic (row 0's seeded history copied on the device to the other rows)",
           "config": {"workload": "%s: %s decode_step_batch, B=%d, contexts U[%d,%d], greedy, %d layers" % (
               args.workload, shape.name, B, args.ctx_lo, args.ctx_hi, shape.n_layers),
               "batch": B, "contexts": [int(c) for c in ctx_main], "kv_format": kv_format,
               "parallelism": "single GPU"},
           "achieved_hbm_GBps": round(step_gbps, 1), "step_bytes": step_bytes,
           "hbm_frac_step": round(step_gbps / HBM_PEAK_GBPS, 4),
           "roofline": roofline, "cpu_baseline": cpu, "parity_first_step": parity, "sweep": sweep_out,
           "kernel_breakdown": breakdown, "sampling": sampling}
    eng.close()
    if args.workload == "llama8b-b8" and not args.no_extras:
        del eng, weights, logits
        torch.cuda.empty_cache()
        out["extras"] = run_extras(args)
    print(json.dumps(out), flush=True)


def host_cores():
    """(host cores this process may run on, BLAS threads numpy uses)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    return cores, blas


# compact runs of the other workloads folded into the default line: each is its own bench.py process
# (fresh device memory), with a bounded oracle sample for parity
EXTRAS = [
    ("mistral7b_int4_b8", ["--workload", "mistral7b-int4", "--steps", "32", "--warmup", "4", "--sweep", "",
                           "--no-breakdown", "--parity-rows", "2"]),
    ("prefill_16seg", ["--workload", "prefill", "--steps", "4", "--warmup", "1", "--no-breakdown"]),
    ("llama8b_long_32k_b8", ["--workload", "llama8b-long", "--steps", "16", "--warmup", "2", "--no-breakdown",
                             "--parity-rows", "1", "--fill", "copy"]),
]


def run_extras(args):
    import subprocess
    res = {}
    for name, extra in EXTRAS:
        cmd = [sys.executable, os.path.abspath(__file__)] + extra
        log("extra %s: %s" % (name, " ".join(extra)))
        t0 = time.time()
        try:
            p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=None, text=True, timeout=400)
            line = [l for l in p.stdout.splitlines() if l.startswith("{")][-1] if p.returncode == 0 else None
        except subprocess.TimeoutExpired:
            line, p = None, None
        if line is None:
            res[name] = {"error": "rc %s" % (p.returncode if p is not None else "timeout")}
            continue
        d = json.loads(line)
        rf = d.get("roofline") or {}
        res[name] = {"value": d["value"], "unit": d["unit"], "ms_per_step": d["ms_per_step"], "steps": d["steps"],
                     "workload": d["config"]["workload"], "data": d.get("data"),
                     "hbm_frac_step": d.get("hbm_frac_step"),
                     "roofline": {k: rf.get(k) for k in ("bound", "achieved", "peak", "unit", "frac", "traffic",
                                                         "kernel", "avg_launch_us", "trace_avg_launch_us",
                                                         "frac_at_trace_avg")},
                     "parity": d.get("parity_first_step") or d.get("parity_last_logits"),
                     "cpu_baseline": d.get("cpu_baseline"), "wall_s": round(time.time() - t0, 1)}
        log("extra %s: %s" % (name, json.dumps(res[name])))
    return res


def run_prefill(args, wl, torch, cbd, synth):
    """prefill_segmented of 16 prompts into fresh slabs, timed over `steps` calls; the 16 slabs are
    allocated before and freed after each call inside the timed loop (host bookkeeping only)."""
    shape = synth.SHAPES[wl["shape"]]
    K = args.batch
    lens = [int(x) for x in synth.uniform_lengths(wl["hist_seed"], K, args.ctx_lo, args.ctx_hi)]
    T = sum(lens)
    V = shape.vocab
    log("prefill: generating %s weights; %d segments, %d tokens" % (shape.name, K, T))
    weights = synth.make_weights(shape, seed=0)
    gran = 256
    arena = sum((l + gran - 1) // gran * gran for l in lens) * shape.kv_bytes_per_token()
    eng = cbd.Engine(weights, arena_bytes=arena, max_batch=64, max_prefill_tokens=T, max_segments=K,
                     max_position=max(lens) + gran)
    dev = torch.device("cuda:0")
    prompts = synth.prompts(wl["hist_seed"] + 1, lens, V)
    toks = torch.from_numpy(np.concatenate(prompts).astype(np.int32)).to(dev)
    logits = torch.empty((K, V), dtype=torch.float32, device=dev)
    nxt = torch.empty(K, dtype=torch.int32, device=dev)

    def one():
        ids = [eng.alloc(l) for l in lens]
        eng.prefill_segmented(ids, lens, toks, logits, nxt)
        return ids

    for _ in range(args.warmup):
        for i in one():
            eng.free(i)
    torch.cuda.synchronize()
    rk = wl["roofline"]
    eng.profile_begin([rk], max_launches=shape.n_layers * args.steps + 64)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for i in one():
            eng.free(i)
    torch.cuda.synchronize()
    secs = time.perf_counter() - t0
    prof = eng.profile_end()
    ms_call = secs * 1e3 / args.steps
    tokps = T * args.steps / secs
    gu = prof[rk]
    avg_ms = gu["total_ms"] / gu["launches"]
    flops_launch = gu["flops"] / gu["launches"]
    achieved = flops_launch / (avg_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS_BF16, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_PEAK_TFLOPS_BF16, 4), "traffic": None,
                "kernel": "dense_gemm_kernel: gate/up + SwiGLU over the %d prefill tokens (256 x 128 tiles), %s" % (
                    T, shape.name),
                "flops_per_launch": flops_launch, "mfma_flops_per_launch": 2 * flops_launch,
                "avg_launch_us": round(avg_ms * 1e3, 2), "launches": gu["launches"]}
    log("prefill: %.1f tok/s, %.2f ms per call; gate/up %.1f us -> %.0f TFLOP/s (%.0f on the matrix cores)" % (
        tokps, ms_call, avg_ms * 1e3, achieved, 2 * achieved))

    breakdown = None
    if not args.no_breakdown:
        eng.profile_begin(cbd.KERNEL_KINDS, max_launches=shape.n_layers * 12 + 16)
        for i in one():
            eng.free(i)
        torch.cuda.synchronize()
        p = eng.profile_end()
        breakdown = {k: {"ms": round(v["total_ms"], 4),
                         "TFLOPs": round(v["flops"] / (v["total_ms"] * 1e-3) / 1e12, 1) if v["flops"] else None,
                         "launches": v["launches"]} for k, v in p.items()}
        log("breakdown (event-timed, one call): %s" % json.dumps(breakdown))

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        from oracle import OracleModel
        cores, blas = host_cores()
        j = int(np.argmin(lens))  # the shortest segment: a bounded sample of the same workload
        got = logits[j].cpu().numpy().astype(np.float64)
        log("cpu baseline: oracle prefill of segment %d (%d tokens, all %d layers + lm_head)" % (j, lens[j],
                                                                                               shape.n_layers))
        orc = OracleModel(weights)
        sid = orc.new_sequence()
        c0 = time.perf_counter()
        ref = orc.prefill(sid, prompts[j].astype(np.int64))
        csecs = time.perf_counter() - c0
        cpu = {"value": round(lens[j] / csecs, 3), "unit": "tok/s", "cores": int(cores), "blas_threads": int(blas),
               "kind": "oracle",
               "sample": "prefill of the shortest of the 16 segments (%d tokens, float64, all 32 layers + lm_head), "
                         "%.1f s" % (lens[j], csecs)}
        err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        parity = {"segment": j, "tokens": lens[j], "max_rel_err": err, "tol": 1e-2,
                  "greedy_match": bool(int(np.argmax(got)) == int(np.argmax(ref)))}
        log("cpu baseline %.2f s; parity %s" % (csecs, parity))

    out = {"metric": "prefill_segmented tok/s, 8B-shape bf16 (16 prompts, lengths U[64,1024])", "value": round(tokps, 1),
           "unit": "tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_call, 3),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "prefill: %s prefill_segmented, K=%d prompts, lengths U[%d,%d] (seed %d), T=%d tokens, "
                                  "%d layers, fresh slabs" % (shape.name, K, args.ctx_lo, args.ctx_hi, wl["hist_seed"], T,
                                                              shape.n_layers),
                      "segments": lens, "parallelism": "single GPU"},
           "roofline": roofline, "cpu_baseline": cpu, "parity_last_logits": parity, "kernel_breakdown": breakdown}
    eng.close()
    print(json.dumps(out), flush=True)


def run_continuous(args, wl, torch, cbd, synth):
    """Continuous batching over the C ABI: admission with a segmented prefill, one batched decode step
    per tick over every live row, retirement between steps (no host synchronisation in the loop)."""
    shape = synth.SHAPES[wl["shape"]]
    caps = [int(x) for x in args.sweep.split(",") if x.strip()]
    V, kv_tok = shape.vocab, shape.kv_bytes_per_token()
    w_bytes = shape.streamed_params() * 2
    log("continuous: generating %s weights" % shape.name)
    weights = synth.make_weights(shape, seed=0)
    gran = 256
    max_ctx = args.ctx_hi + 512
    cap_tokens = (max_ctx + gran - 1) // gran * gran
    max_cap = max(caps)
    eng = cbd.Engine(weights, arena_bytes=(max_cap + 16) * cap_tokens * kv_tok, max_batch=64,
                     max_prefill_tokens=16384, max_segments=16, max_position=cap_tokens)
    dev = torch.device("cuda:0")
    logits = torch.empty((64, V), dtype=torch.float32, device=dev)
    pf_logits = torch.empty((16, V), dtype=torch.float32, device=dev)
    next_b = torch.empty(64, dtype=torch.int32, device=dev)
    pf_next = torch.empty(16, dtype=torch.int32, device=dev)
    tok_by_sid = torch.zeros(4096, dtype=torch.int32, device=dev)
    results = {}
    for cap in caps:
        n_req = 4 * cap + 8
        rng = np.random.Generator(np.random.PCG64(1000 + cap))
        plens = synth.uniform_lengths(2000 + cap, n_req, args.ctx_lo, args.ctx_hi).astype(int)
        glens = synth.uniform_lengths(3000 + cap, n_req, 64, 512).astype(int)
        prompts = synth.shared_prefix_prompts(4000 + cap, plens, V, prefix_len=1024)
        # arrivals in decode ticks: exponential gaps with mean E[gen] / (1.25 cap)
        arrive = np.cumsum(rng.exponential(288.0 / (1.25 * cap), size=n_req))
        arrive -= arrive[0]
        waiting, live = 0, []  # live: [sid, generated, target, context]
        pending = []  # admitted, prompt not yet fully prefilled: [sid, request, tokens done]
        holder = None
        if args.share_prefix:
            # the common prefix, prefilled once; a joiner forks min(L - 1, 1024) of its positions
            holder = eng.alloc(1025)
            eng.prefill_segmented([holder], [1024], torch.from_numpy(prompts[int(np.argmax(plens))][:1024]
                                                                     .astype(np.int32)).to(dev),
                                  pf_logits[:1], pf_next[:1])
        dec_ev, pf_ev = [], []
        dec_rows = pf_tokens = done = 0
        max_stall_ms = 0.0
        step_bytes = 0.0
        tick = 0
        chunk = args.prefill_chunk if args.prefill_chunk > 0 else 16384
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        while done < n_req:
            while waiting < n_req and arrive[waiting] <= tick and len(live) + len(pending) < cap:
                need = int(plens[waiting] + glens[waiting])
                shared = min(int(plens[waiting]) - 1, 1024) if holder is not None else 0
                try:
                    sid = eng.fork(holder, shared, need) if shared else eng.alloc(need)
                except cbd.CbdError:
                    break  # arena full: the request waits
                pending.append([sid, waiting, shared])
                waiting += 1
            # one prefill call per tick: the pending prompts in arrival order, at most `chunk` tokens in
            # all (a prompt may continue over several ticks; --prefill-chunk 0: whole prompts)
            segs, budget = [], chunk
            for q in pending:
                if len(segs) == 16 or budget == 0:
                    break
                rest = int(plens[q[1]]) - q[2]
                if args.prefill_chunk <= 0 and rest > budget:
                    break
                take = min(rest, budget)
                segs.append((q, take))
                budget -= take
            if segs:
                toks = torch.from_numpy(np.concatenate([prompts[q[1]][q[2]:q[2] + n] for q, n in segs])
                                        .astype(np.int32)).to(dev)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                eng.prefill_segmented([q[0] for q, _ in segs], [n for _, n in segs], toks,
                                      pf_logits[:len(segs)], pf_next[:len(segs)])
                e1.record()
                pf_ev.append((e0, e1))
                sids = torch.tensor([q[0] for q, _ in segs], dtype=torch.int64, device=dev)
                tok_by_sid.index_copy_(0, sids, pf_next[:len(segs)])
                for q, n in segs:
                    q[2] += n
                    pf_tokens += n
                    if q[2] == int(plens[q[1]]):  # prompt complete: the last chunk's argmax is token 1
                        live.append([q[0], 1, int(glens[q[1]]), int(plens[q[1]])])
                pending = [q for q in pending if q[2] < int(plens[q[1]])]
            if live:
                ids = [r[0] for r in live]
                idx = torch.tensor(ids, dtype=torch.int64, device=dev)
                last = tok_by_sid.index_select(0, idx)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                eng.decode_step_batch(ids, last, logits[:len(ids)], next_b[:len(ids)])
                e1.record()
                dec_ev.append((e0, e1))
                tok_by_sid.index_copy_(0, idx, next_b[:len(ids)])
                dec_rows += len(ids)
                step_bytes += w_bytes + sum(r[3] + r[1] for r in live) * kv_tok + len(ids) * kv_tok
                for r in live:
                    r[1] += 1
                keep = []
                for r in live:
                    if r[1] >= r[2]:
                        eng.free(r[0])
                        done += 1
                    else:
                        keep.append(r)
                live = keep
                tick += 1
            elif waiting < n_req and not segs and not pending:
                tick = max(tick + 1, int(np.ceil(arrive[waiting])))
        if holder is not None:
            eng.free(holder)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        dec_ms = sum(a.elapsed_time(b) for a, b in dec_ev)
        pf_ms = sum(a.elapsed_time(b) for a, b in pf_ev)
        max_stall_ms = max([a.elapsed_time(b) for a, b in pf_ev] + [0.0])
        gen = int(glens.sum())
        results[str(cap)] = {
            "requests": n_req, "decode_steps": len(dec_ev), "mean_live_rows": round(dec_rows / max(1, len(dec_ev)), 2),
            "decode_tok_s": round(dec_rows / (dec_ms * 1e-3), 1), "decode_ms": round(dec_ms, 1),
            "prefill_calls": len(pf_ev), "prefill_tokens": pf_tokens, "prefill_ms": round(pf_ms, 1),
            "longest_prefill_call_ms": round(max_stall_ms, 1),
            "prefill_tok_s": round(pf_tokens / (pf_ms * 1e-3), 1) if pf_ms else None,
            "wall_tok_s": round(gen / wall, 1), "wall_s": round(wall, 2),
            "decode_GBps": round(step_bytes / (dec_ms * 1e-3) / 1e9, 1),
            "prefix_shared": bool(args.share_prefix)}
        log("cap %d: %s" % (cap, json.dumps(results[str(cap)])))
    top = results[str(max(caps))]
    out = {"metric": "continuous batching: decode-only aggregate tok/s at batch cap %d, 8B-shape bf16" % max(caps),
           "value": top["decode_tok_s"], "unit": "tok/s", "n_gpus": 1, "steps": top["decode_steps"], "warmup": 0,
           "ms_per_step": round(top["decode_ms"] / max(1, top["decode_steps"]), 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "continuous: %s, caps %s, Poisson arrivals (offered 1.25 x cap), prompts U[%d,%d] "
                                  "with a 1024-token shared prefix, generation U[64,512], %d requests per cap = 4 cap + 8; "
                                  "admission %s%s" % (shape.name, caps, args.ctx_lo, args.ctx_hi, 4 * max(caps) + 8,
                                                      "in chunks of at most %d tokens per tick" % args.prefill_chunk
                                                      if args.prefill_chunk > 0 else "of whole prompts",
                                                      "; joiners fork the shared prefix from one prefilled sequence "
                                                      "(kvslab_fork)" if args.share_prefix else ""),
                      "parallelism": "single GPU"},
           "caps": results}
    eng.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
