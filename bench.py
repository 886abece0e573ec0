"""Decode-megakernel benchmark: forward passes/s on the Llama-1B-shaped
batch-1 decode (16 layers, hidden 2048, 32/8 heads, head_dim 64, SwiGLU 8192,
vocab 128256, tied embeddings, bf16 weights ~N(0, 0.02), KV cache prefilled
with bf16 N(0,1) up to position 1024, decode from position 1024).

One "step" is one decoder forward pass (one persistent kernel launch),
enqueued back to back with the on-device token/position advance, inputs
resident in HBM.  Prints one JSON line with the headline number, the HBM
roofline of the megakernel, the CPU-oracle baseline, and extras (the
multi-launch build of the same ops, the flag-synchronised variant, the
homogeneous engine, batched decode of 16 sequences with context lengths
512..4096 on the matrix cores, the grid-barrier microbenchmark and the
streaming-read probe).

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def bytes_per_pass(shape, passes):
    """Algorithmic HBM bytes of one pass, averaged over `passes` (each the
    list of the batch's positions in that pass): every bf16 parameter the
    pass streams, once for the whole batch (one vocab x hidden matrix: the
    LM head, which is the embedding matrix when tied; an untied embedding
    matrix is not streamed, only one row per sequence is gathered); per
    sequence, the keys and values of its cached positions read, the new
    position's keys/values written, fp32 logits written and the token's
    embedding row read."""
    s = shape
    d, L, H = s.head_dim, s.n_layers, s.hidden
    params = L * (H * (s.n_q_heads + 2 * s.n_kv_heads) * d + s.n_q_heads * d * H + 3 * H * s.ffn + 2 * H) \
        + s.vocab * H + H
    kv_b = L * s.n_kv_heads * d * 2 * 2  # bytes per cached position (keys + values)
    total = 0.0
    for ps in passes:
        total += 2 * params + sum(p * kv_b + kv_b + 4 * s.vocab + 2 * H for p in ps)
    return total / len(passes)


COPY_PROBE_BYTES = 256 << 20


def host_facts():
    """CPU model, logical CPU count and RAM of the host the baseline ran on."""
    model, mem_kb = "unknown", 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    mem_kb = int(line.split()[1])
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "ram_gib": round(mem_kb / 2 ** 20, 1)}


def kernel_source_digest() -> str:
    """SHA-256 over the HIP/C++ sources of the library (identifies the kernel build)."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "persistent_megakernel_decode_02_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".h", ".hip", ".cpp")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, mode: str):
    """HBM bytes per launch from the committed counter summary of this kernel
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size), or None when
    there is none or the kernel sources changed since it was taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"traffic_{workload}_{mode}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources") != kernel_source_digest():
        return None
    return round(float(kv["hbm_bytes_per_launch"]))


def run_workload(si, engine, mk, wl, gw, dev, stream, k, w_, log, exec_mode, sync_mode, label):
    """Time k decode passes of workload `wl` (after w_ untimed ones) on the
    given engine; returns a summary dict."""
    import torch
    s, B = wl.shape, wl.batch
    pos0 = wl.positions0(0)
    max_ctx = max(wl.max_ctx, max(pos0) + max(k, w_))
    t0 = time.time()
    kv = si.make_kv_cache(s, B, max_ctx, pos0, master=0).to(dev)
    first = si.workload_tokens(wl, 0)[:B]
    if len(first) < B:
        first = (first * B)[:B]
    log(f"[bench] {wl.name} inputs ready in {time.time() - t0:.1f}s")
    tokens = torch.tensor(first, dtype=torch.int32, device=dev)
    positions = torch.tensor(pos0, dtype=torch.int32, device=dev)
    logits = torch.empty((B, s.vocab), dtype=torch.float32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    eng = engine.Engine(s, gw, max_batch=B, max_ctx=max_ctx, exec_mode=exec_mode, sync_mode=sync_mode,
                        stream=stream)
    try:
        for _ in range(w_):
            eng.step(tokens, positions, kv, logits, nxt, advance=True)
        tokens.copy_(torch.tensor(first, dtype=torch.int32))
        positions.copy_(torch.tensor(pos0, dtype=torch.int32))
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(k):
            eng.step(tokens, positions, kv, logits, nxt, advance=True)
        e1.record(stream)
        torch.cuda.synchronize()
        rc, det = eng.device_error()
        if rc != 0:
            raise RuntimeError(f"device error {rc} ({mk.mk_strerror(rc)}) detail {det}")
        ms = e0.elapsed_time(e1) / k
        info = eng.info
    finally:
        eng.close()
    del kv
    bpp = bytes_per_pass(s, [[p + t for p in pos0] for t in range(k)])
    log(f"[bench] {wl.name} ({label}): {k} passes in {ms * k:.3f} ms")
    return {"workload": wl.name, "batch": B, "exec": label, "passes": k,
            "passes_per_s": round(1000.0 / ms, 2), "tokens_per_s": round(1000.0 * B / ms, 1),
            "ms_per_pass": round(ms, 5), "bytes_per_pass": bpp,
            "hbm_frac": round(bpp / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "kv_splits": info.kv_splits,
            "context_lengths": [min(pos0), max(pos0)]}


def gpu_weights(si, s, dev, seed):
    """Random-init bf16 weights of shape `s` drawn on the device (N(0, 0.02),
    norm gains 1): the timing-only configurations whose weights are too
    large to draw on the host in the time a benchmark run allows."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)

    def normal(shape):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)

    shapes = si.layer_tensor_shapes(s)
    out = {"embed": normal((s.vocab, s.hidden)), "lm_head": None if s.tied else normal((s.vocab, s.hidden)),
           "final_norm": torch.ones(s.hidden, dtype=torch.bfloat16, device=dev)}
    out["layers"] = [{name: (torch.ones(shapes[name], dtype=torch.bfloat16, device=dev) if name.endswith("norm")
                             else normal(shapes[name])) for name in si.LAYER_TENSORS} for _ in range(s.n_layers)]
    return out


def kernel_name(mode: str, per_launch: int) -> str:
    """The kernel that runs a mode's passes (the one profiled for it)."""
    if mode in ("flat-counter", "flat-flag", "flat-sentinel"):
        sent = "_sent" if mode == "flat-sentinel" else ""
        return f"mk_mega{sent}_steps_kernel" if per_launch > 1 else f"mk_mega{sent}_kernel"
    return {"multi": "mk_role_level_kernel", "flat-levels": "mk_flat_level_kernel", "queue-flag": "mk_queue_kernel",
            "stream-counter": "mk_stream_kernel", "stream-flag": "mk_stream_kernel"}.get(mode, "mk_role_mega_kernel")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama1b_pos1024")
    ap.add_argument("--mode", default=None,
                    choices=["mega-counter", "mega-flag", "mega-sentinel", "multi", "flat-counter", "flat-flag",
                             "flat-sentinel", "flat-levels", "queue-flag", "stream-counter", "stream-flag"],
                    help="execution / synchronisation scheme of the headline number (default: flat-sentinel, "
                         "the homogeneous engine polling data sentinels, at batch 1; flat-counter otherwise)")
    ap.add_argument("--trace", default=None, help="write a per-instruction trace of one pass (npz) here")
    ap.add_argument("--trace-passes", type=int, default=4, help="traced passes run back to back (the last is kept)")
    ap.add_argument("--kv-splits", type=int, default=0, help="attention key-range splits (0: planner default)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run one 256 MiB device copy (the scale reference for HBM byte counters)")
    ap.add_argument("--steps-per-launch", type=int, default=1,
                    help="greedy passes per launch of the headline mode (> 1: multi-token persistent decode, "
                         "homogeneous engine only)")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-8b", action="store_true", help="skip the Llama-8B line of the extras")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the decode megakernel path "
                                   "is single-GPU (a sharded layout is designed, not built)", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import synth_inputs as si
    from persistent_megakernel_decode_02_amd import engine, mk

    mk.load_library()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(3)
    dev = "cuda:0"
    wl = si.WORKLOADS[args.workload]
    s = wl.shape
    B = wl.batch
    if args.mode is None:
        args.mode = "flat-sentinel" if B == 1 else "flat-counter"
    K, W = args.steps, args.warmup
    # passes restart from the first position after the warmup (and before a
    # trace), so the workload's own context bound holds whenever it covers them
    max_ctx = max(wl.max_ctx, max(wl.positions0(0)) + max(K, W, args.trace_passes))
    log = lambda *a: print(*a, file=sys.stderr, flush=True)

    t0 = time.time()
    w = si.make_weights(s, master=0)
    gw = engine.to_gpu(w, dev)
    pos0 = wl.positions0(0)
    kv_cpu = si.make_kv_cache(s, B, max_ctx, pos0, master=0)
    kv = kv_cpu.to(dev)
    first = si.workload_tokens(wl, 0)[:B]
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s ({args.workload})")

    stream = torch.cuda.current_stream()
    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {COPY_PROBE_BYTES} bytes read and written")
        del src, dst
    tokens = torch.tensor(first, dtype=torch.int32, device=dev)
    positions = torch.tensor(pos0, dtype=torch.int32, device=dev)
    logits = torch.empty((B, s.vocab), dtype=torch.float32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)

    def timed(exec_mode, sync_mode, k, w_, chunk=1, graph=False):
        """k passes (after w_ warmup passes) as launches of `chunk` greedy
        steps each (mk_decode_steps when chunk > 1), or as replays of one
        captured step (graph: MK_EXEC_FLAT_MULTI)."""
        eng = engine.Engine(s, gw, max_batch=B, max_ctx=max_ctx, kv_splits=args.kv_splits, sync_mode=sync_mode,
                            exec_mode=exec_mode, stream=stream)
        lg_many = nx_many = None
        if chunk > 1:
            lg_many = torch.empty((chunk, B, s.vocab), dtype=torch.float32, device=dev)
            nx_many = torch.empty((chunk, B), dtype=torch.int32, device=dev)

        g = eng.graph(tokens, positions, kv, logits, nxt, advance=True) if graph else None

        def run(n):
            if g is not None:
                for _ in range(n):
                    g.launch()
            elif chunk == 1:
                for _ in range(n):
                    eng.step(tokens, positions, kv, logits, nxt, advance=True)
            else:
                for i in range(0, n, chunk):
                    eng.steps(tokens, positions, kv, lg_many, nx_many, min(chunk, n - i))
        try:
            tokens.copy_(torch.tensor(first, dtype=torch.int32))
            positions.copy_(torch.tensor(pos0, dtype=torch.int32))
            run(w_)
            rc, det = eng.device_error()
            if rc != 0:
                raise RuntimeError(f"device error {rc} ({mk.mk_strerror(rc)}) detail {det}")
            tokens.copy_(torch.tensor(first, dtype=torch.int32))
            positions.copy_(torch.tensor(pos0, dtype=torch.int32))
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run(k)
            e1.record(stream)
            torch.cuda.synchronize()
            rc, det = eng.device_error()
            if rc != 0:
                raise RuntimeError(f"device error {rc} ({mk.mk_strerror(rc)}) detail {det}")
            ms = e0.elapsed_time(e1)
            if args.trace and (exec_mode, sync_mode) == modes[args.mode]:
                tr = torch.zeros(eng.n_instr * 8 + 16, dtype=torch.int64, device=dev)
                mk.mk_ctx_set_trace(eng.ctx, tr.data_ptr(), eng.n_instr, stream.cuda_stream)
                tokens.copy_(torch.tensor(first, dtype=torch.int32))
                positions.copy_(torch.tensor(pos0, dtype=torch.int32))
                for _ in range(args.trace_passes):  # back to back, as in the timed loop; the last one is kept
                    eng.step(tokens, positions, kv, logits, nxt, advance=True)
                torch.cuda.synchronize()
                mk.mk_ctx_set_trace(eng.ctx, None, 0, stream.cuda_stream)
                descs = mk.mk_plan_export(eng.plan)
                arr = np.array([(d.cu, d.slot, d.op, d.layer, d.level, d.r0, d.r1, d.split) for d in descs])
                np.savez(args.trace, desc=arr, t=tr[: eng.n_instr * 8].cpu().numpy().reshape(-1, 8))
            return ms, eng.info
        finally:
            if g is not None:
                g.close()
            eng.close()

    modes = {"mega-counter": (mk.MK_EXEC_MEGA, mk.MK_SYNC_COUNTER), "mega-flag": (mk.MK_EXEC_MEGA, mk.MK_SYNC_FLAG),
             "mega-sentinel": (mk.MK_EXEC_MEGA, mk.MK_SYNC_SENTINEL),
             "multi": (mk.MK_EXEC_MULTI, mk.MK_SYNC_COUNTER),
             "flat-counter": (mk.MK_EXEC_FLAT, mk.MK_SYNC_COUNTER), "flat-flag": (mk.MK_EXEC_FLAT, mk.MK_SYNC_FLAG),
             "flat-sentinel": (mk.MK_EXEC_FLAT, mk.MK_SYNC_SENTINEL),
             "flat-levels": (mk.MK_EXEC_FLAT_MULTI, mk.MK_SYNC_COUNTER),
             "queue-flag": (mk.MK_EXEC_QUEUE, mk.MK_SYNC_FLAG),
             "stream-counter": (mk.MK_EXEC_STREAM, mk.MK_SYNC_COUNTER),
             "stream-flag": (mk.MK_EXEC_STREAM, mk.MK_SYNC_FLAG)}
    spl = max(1, args.steps_per_launch)
    ms, info = timed(*modes[args.mode], K, W, spl)
    log(f"[bench] {args.mode}: {K} passes in {ms:.3f} ms ({spl} per launch)")
    ms_per = ms / K
    passes_s = 1000.0 / ms_per * 1.0
    bpp = bytes_per_pass(s, [[p + t for p in pos0] for t in range(K)])
    achieved = bpp / (ms_per * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(args.workload, args.mode),
            "kernel": kernel_name(args.mode, spl),
            "bytes_per_launch": bpp * spl if args.mode not in ("multi", "flat-levels") else None}

    extras = {"plan": {"cus": info.num_cus, "instructions": info.n_instructions, "levels": info.n_levels,
                       "kv_splits": info.kv_splits, "lds_bytes": info.lds_bytes,
                       "block_threads": info.block_threads}}
    if not args.no_extras:
        for name in [m for m in modes if m != args.mode and (B <= 4 or m.startswith(("flat", "queue")))
                     and (B == 1 or not m.startswith("stream"))]:
            ms2, _ = timed(*modes[name], K, W)
            extras[name] = {"passes_per_s": round(1000.0 * K / ms2, 2), "ms_per_pass": round(ms2 / K, 5),
                            "hbm_frac": round(bpp / (ms2 / K * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[bench] {name}: {K} passes in {ms2:.3f} ms")
        # multi-token persistent decode: all K passes in one launch
        for name in ("flat-sentinel", "flat-counter"):
            if B > 1 and name == "flat-sentinel":
                continue
            if name == args.mode and spl == K:
                continue
            ms2, _ = timed(*modes[name], K, W, K)
            extras.setdefault("one_launch", {})[name] = {
                "passes_per_s": round(1000.0 * K / ms2, 2), "ms_per_pass": round(ms2 / K, 5),
                "hbm_frac": round(bpp / (ms2 / K * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "passes_per_launch": K}
            log(f"[bench] {name}: {K} passes in one launch in {ms2:.3f} ms")
        # the homogeneous engine's multi-launch baseline captured as a hipGraph:
        # the same launches without the host's per-launch cost
        if "flat-levels" in extras:
            ms2, _ = timed(*modes["flat-levels"], K, W, graph=True)
            extras["flat-levels-graph"] = {"passes_per_s": round(1000.0 * K / ms2, 2),
                                           "ms_per_pass": round(ms2 / K, 5),
                                           "hbm_frac": round(bpp / (ms2 / K * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"[bench] flat-levels-graph: {K} passes in {ms2:.3f} ms")
            if args.mode.startswith("flat"):
                extras["bubble_us_per_pass"] = round((extras["flat-levels-graph"]["ms_per_pass"] - ms_per) * 1000.0, 2)
                extras["host_launch_us_per_pass"] = round(
                    (extras["flat-levels"]["ms_per_pass"] - extras["flat-levels-graph"]["ms_per_pass"]) * 1000.0, 2)
                extras["launches_per_pass_levels"] = info.n_levels + 1
        if "multi" in extras and args.mode.startswith("mega"):
            extras["bubble_us_per_pass"] = round((extras["multi"]["ms_per_pass"] - ms_per) * 1000.0, 2)
            extras["launches_per_pass_multi"] = info.n_levels
        # batched decode on the same weights: 16 sequences with context
        # lengths 512..4096, projections as MFMA contractions (FLAT engine)
        bw = si.WORKLOADS["llama1b_b16"]
        if bw.shape == s and B != bw.batch:
            extras["batched"] = run_workload(si, engine, mk, bw, gw, dev, stream, min(K, 32), 2, log,
                                             mk.MK_EXEC_FLAT, mk.MK_SYNC_COUNTER, "flat-counter")
            extras["batched_queue"] = run_workload(si, engine, mk, bw, gw, dev, stream, min(K, 32), 2, log,
                                                   mk.MK_EXEC_QUEUE, mk.MK_SYNC_FLAG, "queue-flag")
        # the other one-sequence configurations in the headline mode: the same
        # weights at context 8192, and the Llama-8B shape (weights drawn on the GPU)
        if B == 1 and args.workload == "llama1b_pos1024":
            hm = modes[args.mode]
            w3 = si.WORKLOADS["llama1b_pos8192"]
            extras["c3"] = run_workload(si, engine, mk, w3, gw, dev, stream, 32, 4, log, *hm, args.mode)
            if not args.no_8b:
                w5 = si.WORKLOADS["llama8b_pos2048"]
                t8 = time.time()
                gw8 = gpu_weights(si, w5.shape, dev, 8)
                log(f"[bench] {w5.name} weights drawn on the GPU in {time.time() - t8:.1f}s")
                extras["c5"] = run_workload(si, engine, mk, w5, gw8, dev, stream, 16, 2, log, *hm, args.mode)
                del gw8
                torch.cuda.empty_cache()
        # grid-barrier microbenchmark
        dinfo = mk.mk_device_query(0)
        n = dinfo.num_cus
        scratch = torch.empty(mk.mk_gridsync_scratch_bytes(n) + 256, dtype=torch.uint8, device=dev)
        base = (scratch.data_ptr() + 255) // 256 * 256
        res = torch.zeros(4, dtype=torch.int32, device=dev)
        gs = {}
        nb = 5000
        for v, vname in mk.GRIDSYNC_VARIANTS.items():
            mk.mk_gridsync_bench(v, 20, n, base, res.data_ptr(), stream.cuda_stream)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            mk.mk_gridsync_bench(v, nb, n, base, res.data_ptr(), stream.cuda_stream)
            e1.record(stream)
            torch.cuda.synchronize()
            gs[vname] = round(e0.elapsed_time(e1) * 1000.0 / nb, 3)
        r = res.cpu().tolist()
        extras["gridsync_us_per_barrier"] = gs
        extras["gridsync_blocks"] = n
        extras["gridsync_errors"] = r[0]
        extras["gridsync_timeouts"] = r[1]
        log(f"[bench] gridsync {gs}")
        del scratch
        # streaming-read probe over 4 GiB (well beyond the 256 MiB Infinity Cache)
        nbytes = 4 << 30
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        out = torch.empty(n * 8, dtype=torch.int32, device=dev)
        mk.mk_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), n * 8, stream.cuda_stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        reps = 5
        for _ in range(reps):
            mk.mk_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), n * 8, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        extras["stream_read_gbs"] = round(reps * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        log(f"[bench] stream read {extras['stream_read_gbs']} GB/s")
        del buf

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle as orc
        model = orc.Model(s, w)
        kv_o = si.bf16_bits(kv_cpu).reshape(kv_cpu.shape).copy()
        tok = list(first)
        pos = list(pos0)
        n_done = 0
        t1 = time.time()
        while n_done == 0 or (time.time() - t1 < args.cpu_seconds and n_done < K):
            _, nx = model.step(tok, pos, kv_o, B, max_ctx)
            tok = [int(v) for v in nx]
            pos = [p + 1 for p in pos]
            n_done += 1
        el = time.time() - t1
        cpu = {"value": round(n_done / el, 4), "unit": "passes/s", "cores": orc.num_threads(), "kind": "oracle",
               "sample": f"{n_done} greedy passes of {args.workload} from position {pos0[0]} (fp64 oracle, "
                         f"OpenMP over output rows), {el:.1f} s"}
        cpu.update(host_facts())
        log(f"[bench] cpu oracle {cpu}")

    line = {
        "metric": "forward passes/s at batch 1 (Llama-1B shape) and % of HBM roofline",
        "value": round(passes_s, 2),
        "unit": "passes/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 weights, fp32 accumulate",
        "data": "synthetic (seeded bf16 N(0,0.02) weights, bf16 N(0,1) KV prefill, uniform token ids)",
        "config": {"workload": args.workload, "batch": B, "start_position": pos0[0], "passes": K,
                   "layers": s.n_layers, "hidden": s.hidden, "heads": f"{s.n_q_heads}/{s.n_kv_heads}",
                   "head_dim": s.head_dim, "ffn": s.ffn, "vocab": s.vocab, "tied": s.tied,
                   "exec": args.mode, "passes_per_launch": spl},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
