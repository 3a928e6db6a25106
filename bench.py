#!/usr/bin/env python3
"""Denoise steps/s of one block-diffusion denoising step on one MI355X.

A step is the whole hot path: mixed-mode attention for the canvas (dg_attn_mixed),
the DiffusionSampler step (dg_sampler_step) and the self-conditioning average
(dg_selfcond_embed). Workload: batch-1 global-attention layer, 256-token
bidirectional canvas on a 4096-token committed prefix, 16 query / 8 KV heads x
head_dim 256, sampler over bf16 logits [256 x 262144] with a 128-nat budget,
self-conditioning against a bf16 embedding table [262144 x 2048]. The denoise loop
runs blocks to the convergence rule (argmax stable 3 steps or mean entropy < 0.05
nats, limit 48): every block starts with a random canvas and its logits follow the
synthetic driver sequence (positions settle over 8 steps), so a block converges
after 12 steps and a new block starts. All inputs are synthetic and seeded, and
resident in HBM before the timed region.

Prints one JSON line: whole-job steps/s, per-kernel times with HIP events on the
launch stream, the roofline of the dominant kernel and the CPU oracle's rate on a
bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoise steps/s (256-tok canvas) + attn MFMA util, sampler HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3

# workload sizes
CANVAS, PREFIX, HQ, HKV, D = 256, 4096, 16, 8, 256
VOCAB, EMBED = 262144, 2048
BUDGET, STABLE_K, TAU, STEP_LIMIT = 128.0, 3, 0.05, 48


def algorithmic():
    """Work the method must do per step (allowed query-key pairs, each byte once)."""
    pairs = CANVAS * (PREFIX + CANVAS)  # every canvas query sees the whole prefix and canvas
    attn_flop = 4 * D * HQ * pairs
    attn_bytes = 2 * (2 * CANVAS * HQ * D + 2 * (PREFIX + CANVAS) * HKV * D)  # Q, O, K, V in bf16
    samp_bytes = 2 * CANVAS * VOCAB + 32 * CANVAS  # logits once + per-row outputs
    samp_probs_bytes = 2 * CANVAS * VOCAB  # block-scaled probabilities written for self-conditioning
    sc_flop = 2 * CANVAS * VOCAB * EMBED
    sc_bytes = 2 * (VOCAB * EMBED + CANVAS * VOCAB + CANVAS * EMBED)
    return dict(attn_flop=attn_flop, attn_bytes=attn_bytes, samp_bytes=samp_bytes, samp_probs_bytes=samp_probs_bytes,
                sc_flop=sc_flop, sc_bytes=sc_bytes)


def _blas():
    """The BLAS numpy runs on, and its thread count (threadpoolctl's report)."""
    try:
        import threadpoolctl
        for info in threadpoolctl.threadpool_info():
            if info.get("user_api") == "blas":
                return {"blas": f"{info.get('internal_api')} {info.get('version')}",
                        "blas_threads": info.get("num_threads")}
    except Exception:  # pragma: no cover - reporting only
        pass
    return {"blas": "unknown", "blas_threads": None}


def cpu_baseline(q, k, v, logits_by_step, E, seqs, seed, min_seconds=10.0, max_steps=6, one_core=True):
    """The oracle, as it stands, on whole steps of the same workload (all canvas rows:
    attention, sampler with its state carried from step to step, self-conditioning),
    run until `min_seconds` have passed, on every host core the process may use (BLAS
    and NumPy threads set to that count); then one more step with BLAS on one thread."""
    from oracle.attn import attn_mixed
    from oracle.sampler import sampler_step, init_canvas, CONV_OR
    from oracle.selfcond import selfcond_embed
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    try:
        import threadpoolctl
        limit = threadpoolctl.threadpool_limits
    except ImportError:  # pragma: no cover
        limit = None
    state = {"canvas": init_canvas([(0, CANVAS, seed, 0)], VOCAB), "prev": np.full(CANVAS, -1, np.int64),
             "stable": [0], "t": 0}

    def one_step():
        t = state["t"]
        logits = logits_by_step(t)
        attn_mixed(seqs, -1, q, k, v, HQ, HKV)
        r = sampler_step(logits, [(0, CANVAS, seed, t)], VOCAB, BUDGET, 1, state["canvas"], state["prev"],
                         state["stable"], stable_k=STABLE_K, tau=TAU, step_limit=STEP_LIMIT, combine=CONV_OR)
        state["canvas"], state["prev"], state["stable"] = r["canvas"], r["prev_argmax"], list(r["stable_count"])
        selfcond_embed(E, logits=logits)
        state["t"] = t + 1

    ctx = limit(limits=cores, user_api="blas") if limit else None
    if ctx is not None:
        ctx.__enter__()
    steps = 0
    t0 = time.perf_counter()
    while steps < max_steps and (steps == 0 or time.perf_counter() - t0 < min_seconds):
        one_step()
        steps += 1
    dt = time.perf_counter() - t0
    blas = _blas()
    if ctx is not None:
        ctx.__exit__(None, None, None)
    res = {"value": round(steps / dt, 6), "unit": "steps/s", "cores": cores, "kind": "oracle",
           "sample": f"{steps} whole steps of the same workload (all {CANVAS} canvas rows: attention, sampler "
                     f"with state carried, self-conditioning) in {dt:.1f} s", "cpu": _cpu_model(), **blas}
    if one_core and limit is not None:
        with limit(limits=1, user_api="blas"):
            t1 = time.perf_counter()
            one_step()
            res["one_core_value"] = round(1.0 / (time.perf_counter() - t1), 6)
            res["one_core_note"] = "one more step with BLAS on one thread (NumPy's elementwise work is single-threaded)"
    return res


COUNTERS = os.path.join(ROOT, "profiles", "denoise_step_prefix4096_canvas256_hbm_counters.md")
SELFCOND_SOURCES = ["selfcond.hip", "dg_host.cpp", "dg_common.cuh", "dg_internal.h"]


def counted_traffic():
    """HBM bytes per dg_selfcond_embed call from the committed counter summary (two
    rocprofv3 --pmc passes, FETCH_SIZE and WRITE_SIZE, scaled by a 1 GiB copy), or None
    once the sources the counters were taken from have changed."""
    try:
        with open(COUNTERS) as f:
            fields = dict(line.strip().split(": ", 1) for line in f if line.startswith(("traffic_", "source_")))
        texts = []
        for name in SELFCOND_SOURCES:
            with open(os.path.join(ROOT, "block_denoising_step_amd", "csrc", name)) as f:
                texts.append(f.read())
    except (OSError, ValueError):
        return None
    if fields.get("source_sha256") != code_hash(texts):
        return None
    return int(fields["traffic_bytes_per_call"])


def code_hash(texts):
    """sha256 of source files with // comments, trailing blanks and empty lines removed,
    so that comment edits do not count as kernel changes."""
    import hashlib
    import re
    h = hashlib.sha256()
    for text in texts:
        for line in text.splitlines():
            line = re.sub(r"//.*", "", line).rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def key_range(mode, prefix, num_q, window, i):
    """Allowed keys [lo, hi] of query i of a request (causal: up to itself; bidirectional:
    the whole canvas; a window W keeps keys within W positions, one-sided for causal)."""
    p = prefix + i
    hi = p if mode == 0 else prefix + num_q - 1
    lo = 0
    if window >= 0:
        lo = max(0, p - window)
        hi = min(hi, p + window)
    return lo, hi


def attn_work(seqs, window, hq, hkv, d, esz, kv_esz=None):
    """Algorithmic FLOPs and bytes of one attention call: allowed (query, key) pairs,
    Q and O once, each touched K/V row once per KV head (kv_esz bytes per K/V element:
    1 for an FP8 cache)."""
    kv_esz = esz if kv_esz is None else kv_esz
    pairs, touched, nq = 0, 0, 0
    for s in seqs:
        if s.num_q == 0:
            continue
        los, his = zip(*(key_range(s.mode, s.prefix_len, s.num_q, window, i) for i in range(s.num_q)))
        pairs += sum(h - l + 1 for l, h in zip(los, his))
        touched += max(his) - min(los) + 1  # key ranges of consecutive queries overlap or touch
        nq += s.num_q
    return 4 * d * hq * pairs, esz * 2 * nq * hq * d + kv_esz * 2 * touched * hkv * d


def per_config(path, reps=20, warm=5, no_oracle=False):
    """Median event time of every call of the five workloads, with each call's
    algorithmic rate and its fraction of the binding roof; written to `path` as JSON."""
    import torch
    import block_denoising_step_amd as dg
    from workloads import attn_case, sampler_case, seed_for, TID_Z, TID_SIGMA, TID_E, CAUSAL

    dev = "cuda:0"
    torch.cuda.set_device(0)
    dg.load()
    stream = torch.cuda.current_stream()
    ridge_bf16 = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    ridge_f32 = PEAK_F32_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)

    def med_us(call):
        for _ in range(warm):
            call(stream)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            call(stream)
            e1.record(stream)
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        return t[len(t) // 2] * 1e3

    def entry(us, flop, nbytes, fp32):
        peak_t = PEAK_F32_TFLOPS if fp32 else PEAK_BF16_TFLOPS
        ridge = ridge_f32 if fp32 else ridge_bf16
        tflops = flop / us / 1e6 if flop else 0.0
        gbs = nbytes / us / 1e3
        mfma = flop > 0 and flop / nbytes > ridge
        e = {"us": round(us, 2), "flop": flop, "bytes": nbytes, "tflops": round(tflops, 1), "gbs": round(gbs, 1),
             "bound": ("mfma_f32" if fp32 else "mfma_bf16") if mfma else "hbm"}
        e["frac"] = round(tflops / peak_t if mfma else gbs / PEAK_HBM_GBS, 4)
        return e

    def gen(seed, shape, std=1.0, dtype=torch.bfloat16):
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        return (torch.randn(shape, device=dev, generator=g) * std).to(dtype)

    def gen_logits(cfg, rows, vocab, dtype):
        g = torch.Generator(device=dev)
        g.manual_seed(seed_for(cfg, TID_SIGMA))
        sig = torch.exp(torch.empty(rows, 1, device=dev).uniform_(np.log(0.1), np.log(10.0), generator=g))
        return (gen(seed_for(cfg, TID_Z), (rows, vocab), dtype=torch.float32) * sig).to(dtype)

    out = {"device": torch.cuda.get_device_name(0), "reps": reps, "warmup": warm, "configs": {}}

    def paged_pool(seqs, k, v, B, seed):
        """Each request's rows in whole B-row blocks, the blocks scattered over the pools
        by a seeded permutation: pools, int32 table, paged requests (kv_start = first entry)."""
        from workloads import Seq
        nbs = [-(-(s.prefix_len + s.num_q) // B) for s in seqs]
        total = sum(nbs)
        perm = torch.randperm(total, generator=torch.Generator().manual_seed(seed))
        kp = torch.zeros((total, B) + tuple(k.shape[1:]), device=dev, dtype=k.dtype)
        vp = torch.zeros_like(kp)
        pseqs, b0 = [], 0
        for s, nb in zip(seqs, nbs):
            n = s.prefix_len + s.num_q
            dst = perm[b0:b0 + nb].to(dev)
            pad = nb * B - n
            for src, pool in ((k, kp), (v, vp)):
                rows = src[s.kv_start:s.kv_start + n]
                if pad:
                    rows = torch.cat([rows, torch.zeros((pad,) + tuple(k.shape[1:]), device=dev, dtype=k.dtype)])
                pool[dst] = rows.view((nb, B) + tuple(k.shape[1:]))
            pseqs.append(Seq(s.q_start, s.num_q, b0, s.prefix_len, s.mode))
            b0 += nb
        return kp.view((-1,) + tuple(k.shape[1:])), vp.view((-1,) + tuple(k.shape[1:])), perm.to(dev, torch.int32), pseqs

    def fp8_codes(x, scale):
        """bf16 K or V rows as E4M3 codes, quantized by dg_kv_write into a pool whose
        table is the identity (so the pool is the contiguous layout); rows past the
        input's end stay zero."""
        B = 256
        nb = -(-x.shape[0] // B)
        pool = torch.zeros((nb * B,) + tuple(x.shape[1:]), device=dev, dtype=torch.float8_e4m3fn)
        table = torch.arange(nb, device=dev, dtype=torch.int32)
        dg.dg_kv_write(x, x, pool, pool, [(0, x.shape[0], 0, 0)], table, B, k_scale=scale, v_scale=scale)
        return pool

    def attn_calls(case, variants, paged_block=0, fp8=False):
        dt = torch.bfloat16 if case.bf16 else torch.float32
        esz = 2 if case.bf16 else 4
        q = gen(seed_for(case.cfg, 1), (case.total_q, case.num_q_heads, case.head_dim), dtype=dt)
        k = gen(seed_for(case.cfg, 2), (case.total_kv, case.num_kv_heads, case.head_dim), dtype=dt)
        v = gen(seed_for(case.cfg, 3), (case.total_kv, case.num_kv_heads, case.head_dim), dtype=dt)
        o = torch.empty_like(q)
        res = {}
        for name, seqs, window in variants:
            c = dg.prepare_attn(q, k, v, o, seqs, window, case.num_q_heads, case.num_kv_heads)
            flop, nbytes = attn_work(seqs, window, case.num_q_heads, case.num_kv_heads, case.head_dim, esz)
            res[name] = entry(med_us(c), flop, nbytes, not case.bf16)
            print(f"[per-config] cfg{case.cfg} {name}: {res[name]}", file=sys.stderr, flush=True)
            if paged_block:
                # the same call on a paged cache (blocks of paged_block rows in a shuffled pool)
                kp, vp, table, pseqs = paged_pool(seqs, k, v, paged_block, seed_for(case.cfg, 9))
                c = dg.prepare_attn(q, kp, vp, o, pseqs, window, case.num_q_heads, case.num_kv_heads,
                                    block_table=table, block_size=paged_block)
                pname = f"{name}_paged_block{paged_block}"
                res[pname] = entry(med_us(c), flop, nbytes, not case.bf16)
                print(f"[per-config] cfg{case.cfg} {pname}: {res[pname]}", file=sys.stderr, flush=True)
                del kp, vp, table
        if fp8:
            # the same calls over an FP8 (E4M3) cache: K/V bytes halve, queries and output stay bf16
            sc = 1.0 / 64
            k8, v8 = fp8_codes(k, sc), fp8_codes(v, sc)
            for name, seqs, window in variants:
                c = dg.prepare_attn(q, k8, v8, o, seqs, window, case.num_q_heads, case.num_kv_heads, k_scale=sc,
                                    v_scale=sc)
                flop, nbytes = attn_work(seqs, window, case.num_q_heads, case.num_kv_heads, case.head_dim, esz, 1)
                fname = f"{name}_fp8_kv"
                res[fname] = entry(med_us(c), flop, nbytes, False)
                print(f"[per-config] cfg{case.cfg} {fname}: {res[fname]}", file=sys.stderr, flush=True)
            del k8, v8
        del q, k, v, o
        return res

    def inject_call(name, M=CANVAS, d=EMBED, hidden=2048, V=VOCAB):
        """dg_selfcond_inject at the step's shapes (bf16): two MFMA GEMMs (gate/up and down,
        6 M d hidden flops) and the weights read once (3 d hidden values)."""
        E = gen(seed_for(2, TID_E), (V, d), std=0.02)
        tokens = torch.randint(0, V, (M,), generator=torch.Generator().manual_seed(seed_for(2, 10))).to(dev, torch.int32)
        s = gen(seed_for(2, 11), (M, d))
        wgu = gen(seed_for(2, 12), (d, 2 * hidden), std=d ** -0.5)
        wd = gen(seed_for(2, 13), (hidden, d), std=hidden ** -0.5)
        out = torch.empty(M, d, device=dev, dtype=torch.bfloat16)
        call = dg.prepare_inject(tokens, E, s, wgu, wd, out)
        flop = 6 * M * d * hidden
        nbytes = 2 * (3 * d * hidden + 3 * M * d) + 4 * M
        e = entry(med_us(call), flop, nbytes, False)
        print(f"[per-config] {name}: {e}", file=sys.stderr, flush=True)
        del E
        return e

    def kv_write_call(name, counts, B=256, hkv=8, d=256):
        """dg_kv_write of `counts` new rows per request (each request's rows after a
        4096-row cache in its own table), bf16: reads and writes each K/V byte once."""
        n = sum(counts)
        k_new = gen(seed_for(4, 2), (n, hkv, d))
        v_new = gen(seed_for(4, 3), (n, hkv, d))
        per = [-(-(4096 + c) // B) for c in counts]
        table = torch.randperm(sum(per), generator=torch.Generator().manual_seed(seed_for(4, 9))).to(dev, torch.int32)
        kp = torch.zeros(sum(per) * B, hkv, d, device=dev, dtype=torch.bfloat16)
        vp = torch.zeros_like(kp)
        seqs, src, t0 = [], 0, 0
        for c, nb in zip(counts, per):
            seqs.append((src, c, t0, 4096))
            src += c
            t0 += nb
        call = dg.prepare_kv_write(k_new, v_new, kp, vp, seqs, table, B)
        e = entry(med_us(call), 0, 2 * 2 * n * hkv * d * 2, False)
        print(f"[per-config] {name}: {e}", file=sys.stderr, flush=True)
        return e

    def sampler_and_selfcond(cfg, with_selfcond):
        sc = sampler_case(cfg)
        dt = torch.bfloat16 if sc.bf16 else torch.float32
        esz = 2 if sc.bf16 else 4
        M, V = sc.total_rows, sc.vocab
        lg = gen_logits(cfg, M, V, dt)
        reqs, r0 = [], 0
        for i, n in enumerate(sc.canvases):
            reqs.append((r0, n, 1000 + i, 0))
            r0 += n
        res = {}
        bufs = dg.SamplerBuffers(M, len(reqs), dev, vocab=V if with_selfcond else 0,
                                 probs_dtype=dt if with_selfcond else None)
        c = dg.prepare_sampler(lg, reqs, V, bufs, sc.budget)
        nbytes = esz * M * V + 32 * M + (esz * M * V if with_selfcond else 0)
        res["sampler" + ("_with_probs" if with_selfcond else "")] = entry(med_us(c), 0, nbytes, False)
        if with_selfcond:
            E = gen(seed_for(cfg, TID_E), (V, sc.embed_dim), std=0.02, dtype=dt)
            so = torch.empty(M, sc.embed_dim, device=dev, dtype=dt)
            cs = dg.prepare_selfcond(bufs.probs, E, so, p_scale=bufs.probs_scale)
            flop = 2 * M * V * sc.embed_dim
            nbytes = esz * (V * sc.embed_dim + M * V + M * sc.embed_dim)
            res["selfcond"] = entry(med_us(cs), flop, nbytes, not sc.bf16)
            del E, so
        for k_, v_ in res.items():
            print(f"[per-config] cfg{cfg} {k_}: {v_}", file=sys.stderr, flush=True)
        del lg, bufs
        return res

    c1 = attn_case(1)
    r = attn_calls(c1, [("attn_bidir_w32", c1.seqs, 32), ("attn_causal_w32", c1.with_mode(CAUSAL).seqs, 32)])
    r.update(sampler_and_selfcond(1, True))
    out["configs"]["1"] = r
    c2 = attn_case(2)
    r = attn_calls(c2, [("attn_bidir_global", c2.seqs, -1)], paged_block=256, fp8=True)
    r["kv_write_canvas256"] = kv_write_call("cfg2 kv_write_canvas256", [256])
    r["selfcond_inject_hidden2048"] = inject_call("cfg2 selfcond_inject_hidden2048")
    r.update(sampler_and_selfcond(2, True))
    out["configs"]["2"] = r
    c3 = attn_case(3)
    out["configs"]["3"] = attn_calls(c3, [("attn_bidir_w512", c3.seqs, 512),
                                          ("attn_causal_w512", c3.with_mode(CAUSAL).seqs, 512)])
    c4 = attn_case(4)
    r = attn_calls(c4, [("attn_global_layer", c4.seqs, -1), ("attn_w512_layer", c4.seqs, 512)], paged_block=256,
                   fp8=True)
    r["kv_write_prefill2048_and_commit256"] = kv_write_call("cfg4 kv_write_prefill2048_and_commit256", [2048, 256])
    r.update(sampler_and_selfcond(4, False))
    out["configs"]["4"] = r
    torch.cuda.empty_cache()
    c5 = attn_case(5)
    r = attn_calls(c5, [("attn_bidir_global", c5.seqs, -1)], paged_block=256, fp8=True)
    torch.cuda.empty_cache()
    r.update(sampler_and_selfcond(5, True))
    out["configs"]["5"] = r
    if not no_oracle:
        torch.cuda.empty_cache()
        out["oracle"] = oracle_per_config()
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"[per-config] wrote {path}", file=sys.stderr, flush=True)


def oracle_per_config(rows_per_request=6, cfgs=(1, 2, 3, 4, 5)):
    """The oracle's time for one step of every workload, on the host cores (BLAS on all
    of them). Attention is timed on `rows_per_request` query rows per request, spread
    over the request, and scaled to all its rows by the keys each row sees (the oracle's
    cost per row is proportional to them); the sampler and self-conditioning run whole."""
    from oracle.attn import attn_mixed, key_range as o_key_range
    from oracle.sampler import sampler_step
    from oracle.selfcond import selfcond_embed
    from workloads import attn_case, sampler_case, logits as synth_logits, embed_table, request_seeds
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    try:
        import threadpoolctl
        ctx = threadpoolctl.threadpool_limits(limits=cores, user_api="blas")
    except ImportError:  # pragma: no cover
        ctx = None

    def attn_time(case, window, full):
        """Seconds for the oracle's attention call: timed whole (full), or per request on
        one row and on `rows_per_request` rows, fitted as a fixed part (the request's K/V
        upcast) plus a part proportional to the keys the rows see, and extrapolated."""
        q, k, v = case.tensors()
        if full:
            t0 = time.perf_counter()
            attn_mixed(case.seqs, window, q, k, v, case.num_q_heads, case.num_kv_heads)
            return time.perf_counter() - t0, case.total_q
        est, timed_rows = 0.0, 0
        for s in case.seqs:
            if s.num_q == 0:
                continue
            nk = np.array([hi - lo + 1 for lo, hi in
                           (o_key_range(s.mode, s.prefix_len, s.num_q, window, i) for i in range(s.num_q))], np.float64)
            pick = sorted(set(int(x) for x in np.linspace(0, s.num_q - 1, min(rows_per_request, s.num_q))))
            ts = []
            for rows in ([pick[0]], pick):
                t0 = time.perf_counter()
                attn_mixed([s], window, q, k, v, case.num_q_heads, case.num_kv_heads, rows=[s.q_start + i for i in rows])
                ts.append(time.perf_counter() - t0)
            ka, kb = nk[pick[0]], nk[pick].sum()
            slope = max(0.0, (ts[1] - ts[0]) / (kb - ka)) if kb > ka else ts[1] / kb
            fixed = max(0.0, ts[0] - slope * ka)
            est += fixed + slope * nk.sum()
            timed_rows += len(pick) + 1
        return est, timed_rows

    def samp_sc_time(cfg, with_sc):
        sc = sampler_case(cfg)
        l = synth_logits(cfg, sc.total_rows, sc.vocab, bf16=sc.bf16)
        seeds = request_seeds(cfg, len(sc.canvases))
        reqs, r0 = [], 0
        for i, n in enumerate(sc.canvases):
            reqs.append((r0, n, seeds[i], 0))
            r0 += n
        M = sc.total_rows
        t0 = time.perf_counter()
        sampler_step(l, reqs, sc.vocab, sc.budget, 1, np.zeros(M, np.int64), np.full(M, -1, np.int64),
                     [0] * len(reqs))
        ts = time.perf_counter() - t0
        tsc = 0.0
        if with_sc:
            E = embed_table(cfg, sc.vocab, sc.embed_dim, bf16=sc.bf16)
            t0 = time.perf_counter()
            selfcond_embed(E, logits=l)
            tsc = time.perf_counter() - t0
        return ts, tsc

    res = {"cores": cores, **_blas(), "cpu": _cpu_model(), "configs": {}}
    for cfg in cfgs:
        case = attn_case(cfg)
        parts = {}
        if cfg == 3:
            t, n = attn_time(case, 512, True)
            parts["attn_bidir_w512"] = t
        elif cfg == 4:
            t1, n = attn_time(case, -1, False)
            t2, _ = attn_time(case, 512, False)
            parts["attn_global_layer"], parts["attn_w512_layer"] = t1, t2
        else:
            t, n = attn_time(case, case.window, cfg != 5)
            parts["attn"] = t
        if cfg != 3:
            ts, tsc = samp_sc_time(cfg, cfg != 4)
            parts["sampler"] = ts
            if cfg != 4:
                parts["selfcond"] = tsc
        total = float(sum(parts.values()))
        res["configs"][str(cfg)] = {"seconds_per_step": round(total, 3), "steps_per_s": round(1.0 / total, 5),
                                    "parts_seconds": {k_: round(float(v_), 3) for k_, v_ in parts.items()},
                                    "attention_rows_timed": int(n)}
        print(f"[per-config] oracle cfg{cfg}: {res['configs'][str(cfg)]}", file=sys.stderr, flush=True)
    if ctx is not None:
        ctx.unregister()
    res["sample"] = (f"configs 1-3: whole calls; configs 4 and 5: attention per request on 1 and on "
                     f"{rows_per_request} query rows, fitted as a fixed part plus a part proportional to the keys "
                     "the rows see and extrapolated to every row; sampler and self-conditioning on every row")
    return res


def measure_ceilings(torch, read_sizes=(134217728, 1208991744, 4294967296), copy_bytes=1073741824,
                     reps=20, warm=5, mfma_iters=20000):
    """Achievable ceilings with the in-tree measurement kernels (libdg_probe.so): a streaming
    read at each size in read_sizes (the sampler's logits, the self-conditioning call's
    bytes, 4 GiB), a copy, and back-to-back bf16 MFMAs; the best over a few launch shapes,
    median event time of `reps` launches each."""
    from block_denoising_step_amd import probe
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def med_ms(fn):
        for _ in range(warm):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        return t[len(t) // 2]

    res = {"cus": cus, "reps": reps, "read": [], "copy": None, "mfma_bf16": None}
    big = torch.empty(max(max(read_sizes), 2 * copy_bytes), dtype=torch.uint8, device=dev)
    big[::4096].fill_(1)
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    for nbytes in read_sizes:
        src = big[:nbytes]
        best = None
        for blocks in (cus, cus * 2, cus * 4, cus * 8, cus * 16):
            ms = med_ms(lambda: probe.read(src, sink, blocks))
            gbs = nbytes / ms / 1e6
            if best is None or gbs > best["gbs"]:
                best = {"bytes": nbytes, "blocks": blocks, "us": round(ms * 1e3, 2), "gbs": round(gbs, 1)}
        best["frac_of_8000"] = round(best["gbs"] / PEAK_HBM_GBS, 4)
        res["read"].append(best)
        print(f"[ceilings] read {best}", file=sys.stderr, flush=True)
    half = copy_bytes
    srcb = big[:half]
    dstb = big[half:2 * half]
    best = None
    for blocks in ((cus * 4, cus * 8, cus * 16) if copy_bytes else ()):
        ms = med_ms(lambda: probe.copy(dstb, srcb, blocks))
        gbs = 2 * half / ms / 1e6
        if best is None or gbs > best["gbs_read_plus_write"]:
            best = {"bytes_each_way": half, "blocks": blocks, "us": round(ms * 1e3, 2), "gbs_read_plus_write": round(gbs, 1)}
    if best is not None:
        best["frac_of_8000"] = round(best["gbs_read_plus_write"] / PEAK_HBM_GBS, 4)
        res["copy"] = best
        print(f"[ceilings] copy {best}", file=sys.stderr, flush=True)
    del big
    msink = torch.empty(cus * 2 * 256, dtype=torch.float32, device=dev)
    # operands: N(0, 1) bf16 draws (as a GEMM's inputs vary), or one fixed pair
    g = torch.Generator(device=dev)
    g.manual_seed(214999)
    ops = torch.randn(cus * 2 * 256 * 64, device=dev, generator=g).to(torch.bfloat16)
    for label, o in (("mfma_bf16", ops), ("mfma_bf16_fixed_operands", None)):
        best = None
        for blocks in (cus, cus * 2):
            ms = med_ms(lambda: probe.mfma_bf16(msink, blocks, mfma_iters, ops=o))
            flop = blocks * 4 * mfma_iters * 8 * 2 * 32 * 32 * 16
            tf = flop / ms / 1e9
            if best is None or tf > best["tflops"]:
                best = {"blocks": blocks, "waves_per_cu": 4 * blocks // cus, "iters": mfma_iters,
                        "us": round(ms * 1e3, 2), "tflops": round(tf, 1)}
        best["frac_of_2500"] = round(best["tflops"] / PEAK_BF16_TFLOPS, 4)
        res[label] = best
        print(f"[ceilings] {label} {best}", file=sys.stderr, flush=True)
    return res


def ceilings(path):
    import torch
    torch.cuda.set_device(0)
    res = measure_ceilings(torch)
    res["device"] = torch.cuda.get_device_name(0)
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res), flush=True)


def wait_flag(flags, slot, timeout_s=30.0):
    """Spin until the selection kernel has written slot `slot` of the pinned flag pair
    (the host set it to -1 before enqueueing that step); return the flag."""
    t0 = time.perf_counter()
    n = 0
    while True:
        f = int(flags[slot].item())
        if f >= 0:
            return f
        n += 1
        if n % 4096 == 0 and time.perf_counter() - t0 > timeout_s:
            raise RuntimeError("the converged flag of a step was not written in time")


def block_loop(path, blocks=8, prompt=PREFIX, block_size=256):
    """The block-autoregressive loop on a paged cache, at the step workload's shapes:
    a prefill of `prompt` tokens (K/V written through the block table, one causal pass),
    then `blocks` blocks of denoise steps (canvas draft K/V written, bidirectional
    attention, sampler, self-conditioning) until the convergence rule fires, each
    committed by a causal pass over its 256 tokens, the next canvas placed after it.
    The logits follow the same synthetic settling driver as the step loop, so a block
    takes 12 steps. Writes JSON to `path` and prints one line."""
    import torch
    import block_denoising_step_amd as dg
    from workloads import Seq, embed_table, driver_pool, driver_rows, request_seeds, CAUSAL, BIDIR

    dev = "cuda:0"
    torch.cuda.set_device(0)
    dg.load()
    stream = torch.cuda.current_stream()
    bf = torch.bfloat16

    def gen(seed, shape, std=1.0):
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        return (torch.randn(shape, device=dev, generator=g) * std).to(bf)

    total = prompt + blocks * CANVAS
    nblk = -(-total // block_size)
    table = torch.randperm(nblk, generator=torch.Generator().manual_seed(214091)).to(dev, torch.int32)
    kp = torch.zeros(nblk * block_size, HKV, D, device=dev, dtype=bf)
    vp = torch.zeros_like(kp)
    E = torch.from_numpy(embed_table(2, VOCAB, EMBED, bf16=True)).to(dev).to(bf)
    pool = torch.from_numpy(driver_pool(VOCAB, bf16=True)).to(dev).to(bf)
    step_logits = [pool[torch.from_numpy(driver_rows(t)).to(dev)].contiguous() for t in range(9)]
    seed = request_seeds(2, 1)[0]
    # the model's stand-in: prompt K/V and queries, two alternating canvas drafts, commit rows
    pk, pv, pq = gen(214101, (prompt, HKV, D)), gen(214102, (prompt, HKV, D)), gen(214103, (prompt, HQ, D))
    dk = [gen(214111 + i, (CANVAS, HKV, D)) for i in range(2)]
    dv = [gen(214121 + i, (CANVAS, HKV, D)) for i in range(2)]
    dq = [gen(214131 + i, (CANVAS, HQ, D)) for i in range(2)]
    ck, cv, cq = gen(214141, (CANVAS, HKV, D)), gen(214142, (CANVAS, HKV, D)), gen(214143, (CANVAS, HQ, D))
    out_p = torch.empty(prompt, HQ, D, device=dev, dtype=bf)
    out_c = torch.empty(CANVAS, HQ, D, device=dev, dtype=bf)
    bufs = dg.SamplerBuffers(CANVAS, 1, dev, vocab=VOCAB, probs_dtype=bf)
    sc_out = torch.empty(CANVAS, EMBED, device=dev, dtype=bf)
    flags = torch.zeros(2, dtype=torch.int32, pin_memory=True)
    samp_calls = [dg.prepare_sampler(step_logits[t], [(0, CANVAS, seed, 0)], VOCAB, bufs, BUDGET, stable_k=STABLE_K,
                                     tau=TAU, step_limit=STEP_LIMIT, combine=dg.DG_CONV_OR) for t in range(9)]
    init_call = dg.prepare_sampler(None, [(0, CANVAS, seed, 0)], VOCAB, bufs, BUDGET, flags=dg.DG_INIT_CANVAS,
                                   num_rows=CANVAS)
    sc_call = dg.prepare_selfcond(bufs.probs, E, sc_out, p_scale=bufs.probs_scale)

    def run():
        steps = []
        dg.prepare_kv_write(pk, pv, kp, vp, [(0, prompt, 0, 0)], table, block_size)(stream)
        dg.prepare_attn(pq, kp, vp, out_p, [Seq(0, prompt, 0, 0, CAUSAL)], -1, HQ, HKV, block_table=table,
                        block_size=block_size)(stream)
        prefix, issued = prompt, 0
        for b in range(blocks):
            draft = [dg.prepare_kv_write(dk[i], dv[i], kp, vp, [(0, CANVAS, 0, prefix)], table, block_size)
                     for i in range(2)]
            attn = [dg.prepare_attn(dq[i], kp, vp, out_c, [Seq(0, CANVAS, 0, prefix, BIDIR)], -1, HQ, HKV,
                                    block_table=table, block_size=block_size) for i in range(2)]
            init_call.args._keep[0].seed = (seed + b) & ((1 << 64) - 1)
            init_call(stream)
            t = 0
            while True:
                draft[t % 2](stream)
                attn[t % 2](stream)
                samp = samp_calls[min(t, 8)]
                samp.args._keep[0].step = t
                samp.args._keep[0].seed = (seed + b) & ((1 << 64) - 1)
                slot = issued % 2
                flags[slot] = -1
                samp.args.converged = flags[slot:slot + 1].data_ptr()
                samp(stream)
                sc_call(stream)
                issued += 1
                t += 1
                # this step's flag, written by the selection while its self-conditioning
                # GEMM still has most of the step to run
                if wait_flag(flags, slot) or t >= STEP_LIMIT:
                    break
            steps.append(t)
            dg.prepare_kv_write(ck, cv, kp, vp, [(0, CANVAS, 0, prefix)], table, block_size)(stream)
            dg.prepare_attn(cq, kp, vp, out_c, [Seq(0, CANVAS, 0, prefix, CAUSAL)], -1, HQ, HKV,
                            block_table=table, block_size=block_size)(stream)
            prefix += CANVAS
        torch.cuda.synchronize()
        return steps, issued

    run()  # warm-up pass
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    steps, issued = run()
    elapsed = time.perf_counter() - t0
    res = {"workload": f"block loop on a paged cache: prompt {prompt}, {blocks} blocks of {CANVAS} tokens, "
                       f"16 q / 8 kv heads x 256, vocab {VOCAB}, embed {EMBED}, cache blocks of {block_size} rows",
           "committed_tokens_per_s": round(blocks * CANVAS / elapsed, 1),
           "denoise_steps_per_s": round(issued / elapsed, 1),
           "steps_per_block": steps, "steps_issued": issued, "seconds": round(elapsed, 5),
           "note": "includes the prefill, the commit passes and the host's flag reads"}
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res), flush=True)


def graph_steps(path, args, dg, torch, step, seed, flags):
    """The step loop with every step replayed from a recorded HIP graph: attention, the
    sampler (reading its step from a device counter that the selection advances) and
    self-conditioning, recorded once per (logits buffer, converged-flag slot) pair, so
    the host enqueues one replay per step. Blocks restart with an eager DG_INIT_CANVAS
    call that zeroes the counter; the seed stays the same from block to block (it is a
    recorded argument). Writes JSON to `path` and prints one line."""
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    bufs, step_logits = step.bufs, step.logits
    counter = torch.zeros(1, dtype=torch.int32, device=dev)
    kw = dict(stable_k=STABLE_K, tau=TAU, step_limit=STEP_LIMIT, combine=dg.DG_CONV_OR, step_counter=counter,
              probs=bufs.probs, probs_scale=bufs.probs_scale)
    init = dg.prepare_sampler(None, [(0, CANVAS, seed, 0)], VOCAB, bufs, BUDGET, flags=dg.DG_INIT_CANVAS,
                              num_rows=CANVAS, step_counter=counter)
    side = torch.cuda.Stream()
    graphs = []
    t_rec = time.perf_counter()
    for i, lg in enumerate(step_logits):
        pair = []
        for slot in range(2):
            samp = dg.prepare_sampler(lg, [(0, CANVAS, seed, 0)], VOCAB, bufs, BUDGET, **kw)
            samp.args.converged = flags[slot:slot + 1].data_ptr()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                step.attn()
                samp()
                step.selfcond[i]()
            pair.append((g, samp))
        graphs.append(pair)
    torch.cuda.synchronize()
    t_rec = time.perf_counter() - t_rec
    state = {"t": 0, "issued": 0, "blocks": 0, "spec": 0}

    def start_block():
        init(stream)
        state["t"] = 0

    def one_step():
        """Replay one step and return its converged flag (written by the selection,
        before the step's self-conditioning)."""
        t = state["t"]
        slot = state["issued"] % 2
        flags[slot] = -1
        graphs[min(t, len(graphs) - 1)][slot][0].replay()
        state["issued"] += 1
        state["t"] = t + 1
        return bool(wait_flag(flags, slot))

    def run(n):
        for _ in range(n):
            if one_step() or state["t"] >= STEP_LIMIT:
                state["blocks"] += 1
                start_block()

    start_block()
    run(args.warmup)
    torch.cuda.synchronize()
    b0, s0 = state["blocks"], state["spec"]
    t0 = time.perf_counter()
    run(args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    useful = args.steps - (state["spec"] - s0)
    res = {"mode": "each step replayed from a recorded HIP graph (attention, sampler with a device step counter, "
                   "self-conditioning)",
           "steps_per_s": round(useful / elapsed, 3), "ms_per_step": round(elapsed * 1e3 / useful, 4),
           "steps": args.steps, "speculative_steps": args.steps - useful, "warmup": args.warmup,
           "blocks_in_timed_region": state["blocks"] - b0,
           "graphs": len(graphs) * 2, "record_seconds": round(t_rec, 4),
           "workload": "the default step workload (canvas 256 on prefix 4096, vocab 262144, embed 2048, bf16)"}
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    # the GPU's clock settles over the first tens of milliseconds of sustained load
    # (measured: 24 warm-up steps left part of a slower phase in the timed region, -1.5%)
    ap.add_argument("--warmup", type=int, default=120)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--per-config", metavar="PATH",
                    help="instead of the step loop, time every call of the five workloads and write JSON to PATH")
    ap.add_argument("--block-loop", metavar="PATH",
                    help="instead of the step loop, time the block-autoregressive loop on a paged cache; JSON to PATH")
    ap.add_argument("--ceilings", metavar="PATH",
                    help="instead of the step loop, measure the achievable HBM read/copy and bf16 MFMA ceilings "
                         "with the in-tree measurement kernels; JSON to PATH")
    ap.add_argument("--graph", metavar="PATH",
                    help="instead of the eager step loop, replay each step from a recorded HIP graph; JSON to PATH")
    ap.add_argument("--selfcond-input", choices=("probs", "logits"), default="probs",
                    help="what self-conditioning reads: the sampler's block-scaled probabilities, or the logits "
                         "with the sampler's row statistics")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size kernel for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if args.per_config:
        per_config(args.per_config, no_oracle=args.no_cpu_baseline)
        return
    if args.block_loop:
        block_loop(args.block_loop)
        return
    if args.ceilings:
        ceilings(args.ceilings)
        return

    import torch
    import block_denoising_step_amd as dg
    from block_denoising_step_amd.step import DenoiseStep
    from workloads import attn_case, embed_table, driver_pool, driver_rows, request_seeds

    dev = "cuda:0"
    torch.cuda.set_device(0)
    dg.load()

    # ---- inputs, resident in HBM before timing ---------------------------------------
    case = attn_case(2)
    q_np, k_np, v_np = case.tensors()
    q = torch.from_numpy(q_np).to(dev).to(torch.bfloat16)
    k = torch.from_numpy(k_np).to(dev).to(torch.bfloat16)
    v = torch.from_numpy(v_np).to(dev).to(torch.bfloat16)
    E_np = embed_table(2, VOCAB, EMBED, bf16=True)
    E = torch.from_numpy(E_np).to(dev).to(torch.bfloat16)
    pool_np = driver_pool(VOCAB, bf16=True)
    pool = torch.from_numpy(pool_np).to(dev).to(torch.bfloat16)
    settle = 9  # steps >= 8 read the settled rows: 9 distinct logits tensors cover every step
    step_logits = [pool[torch.from_numpy(driver_rows(t)).to(dev)].contiguous() for t in range(settle)]
    seed = request_seeds(2, 1)[0]
    step = DenoiseStep(q, k, v, case.seqs, -1, HQ, HKV, step_logits, E, BUDGET, STABLE_K, TAU, STEP_LIMIT,
                       combine=dg.DG_CONV_OR, seed=seed, selfcond_input=args.selfcond_input)

    stream = torch.cuda.current_stream()
    # The selection writes each step's converged flag straight into pinned host memory,
    # alternating between two slots so that step t never overwrites the flag of step t-1
    # before the host has read it. The host sets a slot to -1 before the step that
    # writes it is enqueued, then waits for a 0 or 1 there: the flag itself says that the
    # step's selection has run, so neither a copy nor an event (whose record costs about
    # 6 us of GPU time) sits on the stream between steps.
    flags = torch.zeros(2, dtype=torch.int32, pin_memory=True)
    if args.graph:
        graph_steps(args.graph, args, dg, torch, step, seed, flags)
        return

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # issued: steps enqueued. The host enqueues a step, then waits for that step's
    # converged flag, which the selection writes midway through the step (before
    # self-conditioning): the step's GEMM still has most of the step's GPU time to run
    # while the host enqueues the next step (or starts a new block), so the GPU never
    # idles and no step is enqueued that a converged block would throw away.
    state = {"t": 0, "block": 0, "issued": 0, "spec": 0}

    def start_block():
        step.start_block(seed + state["block"], stream)
        state["t"] = 0

    def one_step(ev=None):
        """Enqueue one step and return its converged flag. ev: None, or four events (a
        sample of the timed steps is bracketed by events: each record costs GPU time)."""
        t = state["t"]
        slot = state["issued"] % 2
        flags[slot] = -1
        step.enqueue(t, min(t, settle - 1), stream, converged_ptr=flags[slot:slot + 1].data_ptr(), events=ev)
        state["issued"] += 1
        state["t"] = t + 1
        return bool(wait_flag(flags, slot))

    def run(n, events=None):
        for s_ in range(n):
            if one_step(events[s_] if events is not None else None) or state["t"] >= STEP_LIMIT:
                state["block"] += 1
                start_block()

    start_block()
    run(args.warmup)
    torch.cuda.synchronize()
    # every SAMPLE_EVERY-th timed step is bracketed by events (per-call times, including
    # the roofline kernel's); the others run without any
    SAMPLE_EVERY = 8
    events = [[torch.cuda.Event(enable_timing=True) for j in range(4)] if i % SAMPLE_EVERY == 0 else None
              for i in range(args.steps)]
    blocks0, spec0 = state["block"], state["spec"]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.steps, events)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    blocks = state["block"] - blocks0
    spec = state["spec"] - spec0

    # achievable ceilings, measured after the timed region in the same process: a streaming
    # read of the sampler's and the self-conditioning call's byte counts, bf16 MFMA
    alg0 = algorithmic()
    ceil = measure_ceilings(torch, read_sizes=(alg0["samp_bytes"] // 16 * 16, alg0["sc_bytes"] // 16 * 16),
                            copy_bytes=0, mfma_iters=4000)
    ceil_read = {r["bytes"]: r["gbs"] for r in ceil["read"]}
    samp_ceil = ceil_read[alg0["samp_bytes"] // 16 * 16]
    sc_ceil = ceil_read[alg0["sc_bytes"] // 16 * 16]
    mfma_ceil = ceil["mfma_bf16"]["tflops"]

    sampled = [e for e in events if e is not None]
    attn_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in sampled]))
    samp_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in sampled]))
    sc_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in sampled]))
    alg = algorithmic()
    useful = args.steps - spec
    ms_per_step = elapsed * 1e3 / useful
    value = useful / elapsed

    attn_tflops = alg["attn_flop"] / (attn_ms * 1e-3) / 1e12
    samp_gbs = alg["samp_bytes"] / (samp_ms * 1e-3) / 1e9
    probs_mode = args.selfcond_input == "probs"
    samp_rw_gbs = (alg["samp_bytes"] + alg["samp_probs_bytes"]) / (samp_ms * 1e-3) / 1e9
    sc_gbs = alg["sc_bytes"] / (sc_ms * 1e-3) / 1e9
    sc_tflops = alg["sc_flop"] / (sc_ms * 1e-3) / 1e12

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "batch-1 global-attention denoise step: canvas 256 (bidirectional) on prefix 4096, "
                        "16 q / 8 kv heads x 256; sampler on bf16 logits [256 x 262144], budget 128 nats; "
                        "self-conditioning with bf16 E [262144 x 2048]; blocks run to argmax-stable-3 or "
                        "mean entropy < 0.05 (limit 48)",
            "canvas": CANVAS, "prefix": PREFIX, "q_heads": HQ, "kv_heads": HKV, "head_dim": D,
            "vocab": VOCAB, "embed_dim": EMBED, "blocks_in_timed_region": blocks,
            "selfcond_input": args.selfcond_input,
        },
        "steps_issued": args.steps,
        "speculative_steps": spec,
        "value_note": "every timed step is a useful one: the host reads each step's converged flag as soon as "
                      "the selection writes it (before the step's self-conditioning), so no step is enqueued past a "
                      "converged block",
        "roofline": {
            "kernel": "dg_selfcond_embed (selfcond_gemm_dma + selfcond_reduce)",
            "bound": "hbm",
            "achieved": round(sc_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(sc_gbs / PEAK_HBM_GBS, 4),
            "traffic": counted_traffic(),
            "traffic_unit": "bytes per call",
            "measured_ceiling": sc_ceil,
            "frac_of_measured_ceiling": round(sc_gbs / sc_ceil, 4),
            "ceiling_note": "measured_ceiling: in-tree streaming-read kernel over the same byte count, in this run",
        },
        "kernels": {
            "attn_mixed": {"ms": round(attn_ms, 4), "tflops": round(attn_tflops, 1),
                           "frac_bf16_mfma_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                           "frac_measured_mfma_ceiling": round(attn_tflops / mfma_ceil, 4)},
            "sampler_step": dict({"ms": round(samp_ms, 4), "gbs": round(samp_gbs, 1),
                                  "frac_hbm_peak": round(samp_gbs / PEAK_HBM_GBS, 4),
                                  "frac_measured_read_ceiling": round(samp_gbs / samp_ceil, 4)},
                                 **({"gbs_with_probs_write": round(samp_rw_gbs, 1),
                                     "frac_hbm_peak_with_probs_write": round(samp_rw_gbs / PEAK_HBM_GBS, 4)}
                                    if probs_mode else {})),
            "selfcond_embed": {"ms": round(sc_ms, 4), "gbs": round(sc_gbs, 1), "tflops": round(sc_tflops, 1),
                               "frac_hbm_peak": round(sc_gbs / PEAK_HBM_GBS, 4),
                               "frac_measured_read_ceiling": round(sc_gbs / sc_ceil, 4)},
            "measured_ceilings": {"read_gbs": {str(k_): v_ for k_, v_ in ceil_read.items()},
                                  "mfma_bf16_tflops": mfma_ceil},
            "timing": f"HIP events on the launch stream around each call, on {len(sampled)} of the {args.steps} "
                      f"timed steps (every {SAMPLE_EVERY}th)",
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(q_np, k_np, v_np, lambda t: pool_np[driver_rows(t)], E_np, case.seqs,
                                            seed)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
