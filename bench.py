#!/usr/bin/env python3
"""Benchmark of the DFlash block-drafter proposal pass on one MI355X.

Workload (one step = one decode cycle): 8192 resident context cells, a block
of anchor + 7 masks (block 8) drafted at the next position, greedy
verification against a seeded stand-in target that agrees with each
candidate with probability 0.75, and the commit (fusion + K/V projection) of
the accepted cells plus the anchor -- done by the next cycle's pass (one
launch commits and drafts).  The timed cycles keep their positions in device
words that the verify advances (dflash_draft_block_commit_dev,
dflash_verify_greedy_advance), so no cycle reads from the device; jobs of 26
cycles (about 96 committed tokens) restart at position 8192
(position-addressed cells make rejected drafts harmless).  The same cycle
with host-side positions (one device-to-host read per cycle) and with the
commit as separate calls are reported beside it.

Prints one JSON line.  Inputs are resident in HBM before timing starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CTX = 8192
BLOCK = 8
JOB_TOKENS = 96
JOB_CYCLES = 26   # cycles per job of the device-resident loop (about 96 tokens at p = 0.75)
HBM_PEAK_GBS = 8000.0
METRIC = "DFlash draft passes/sec (ctx 8192, block 8) + achieved HBM GB/s vs peak"


# Stored bytes per weight of the layer matrices: bf16, Q8_0 (32 int8 + fp16
# scale per 32 weights), Q4_0 (16 bytes of nibbles + fp16 scale per 32), Q5_0
# (Q4_0 plus a 4-byte word of fifth bits per 32).
BYTES_PER_WEIGHT = {"bf16": 2.0, "q8_0": 34 / 32, "q4_0": 18 / 32, "q5_0": 22 / 32}


def pass_bytes(n_ctx: int, block: int = BLOCK, fmt: str = "bf16", lm_fmt: str = "bf16") -> int:
    """Algorithmic HBM bytes of one draft pass: every layer matrix (in its
    storage format) and the LM head (bf16 or Q8_0) once, the gains, the
    distinct embedding rows and n_ctx fp16 K/V cells (5 layers x 2 KV heads
    x 256 x K and V)."""
    from block_draft_model_pass_amd import synth as S
    H, D, F = S.HIDDEN, S.HEAD_DIM, S.FFN
    qkv = (S.N_Q_HEADS + 2 * S.N_KV_HEADS) * D * H
    layer = qkv + H * S.N_Q_HEADS * D + 2 * F * H + H * F
    mats = int(round(BYTES_PER_WEIGHT[fmt] * S.N_LAYERS * layer))
    gains = 2 * (S.N_LAYERS * (2 * H + 2 * D) + H)
    lm = int(round(BYTES_PER_WEIGHT[lm_fmt] * S.VOCAB * H)) if block > 1 else 0
    emb = 2 * H * (2 if block > 1 else 1)
    kv = n_ctx * S.N_LAYERS * S.N_KV_HEADS * D * 2 * 2
    return mats + gains + lm + emb + kv


PROFILE = os.path.join(ROOT, "profiles", "k_draft_pass_ctx8192_block8_bf16.md")


def kernel_source_hash() -> str:
    """First 16 hex digits of sha256 over the pass kernel's sources."""
    import hashlib
    h = hashlib.sha256()
    for f in ("pass.hip", "common.h"):
        with open(os.path.join(ROOT, "block_draft_model_pass_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per pass from the committed FETCH_SIZE / WRITE_SIZE counter
    runs, or None when the kernel sources changed since they were taken."""
    import re
    try:
        with open(PROFILE) as fh:
            text = fh.read()
    except OSError:
        return None
    t = re.search(r"^traffic_bytes_per_launch: (\d+)", text, re.M)
    h = re.search(r"^kernel_source_sha256_16: ([0-9a-f]+)", text, re.M)
    if not t or not h or h.group(1) != kernel_source_hash():
        return None
    return int(t.group(1))


def lm_head_bytes() -> int:
    from block_draft_model_pass_amd import synth as S
    return 2 * S.VOCAB * S.HIDDEN


def cpu_baseline(host_w, budget_s: float):
    """The oracle's decode cycle at ctx 8192 / block 8 on the host cores."""

    from block_draft_model_pass_amd import synth
    from oracle import dflash_oracle as O
    w = O.enable_cache(dict(host_w))
    store = O.ContextStore()
    for s in range(0, CTX, 2048):
        taps = synth.make_taps(range(s, s + 2048))
        store.put(*O.project_ctx_kv(w, O.fuse_context(w, taps), s), s)
    K = BLOCK - 1
    p, anchor = CTX, synth.anchor_token(0)
    ck, cv = store.window(p)
    O.draft_block(w, ck, cv, p, anchor, synth.MASK_ID, BLOCK)  # fills the decode cache
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s or n < 2:
        ck, cv = store.window(p)
        ref = O.draft_block(w, ck, cv, p, anchor, synth.MASK_ID, BLOCK)
        tgt = synth.synthetic_target(ref["cand"], n)
        a, nxt = O.verify_greedy(ref["cand"], tgt)
        taps = synth.make_taps(range(p, p + a + 1))
        store.put(*O.project_ctx_kv(w, O.fuse_context(w, taps), p), p)
        p, anchor = p + a + 1, nxt
        n += 1
    dt = time.perf_counter() - t0
    info = host_cpu()
    return {"value": n / dt, "unit": "passes/s", "cores": info["blas_threads"], "kind": "oracle",
            "sample": f"{n} decode cycles (draft + verify + commit) of the fp64 numpy oracle "
                      f"at ctx {CTX}, block {BLOCK}, {dt:.1f} s; weights pre-decoded; "
                      f"{info['model']}, {info['cores']} cores available"}


def host_cpu() -> dict:
    """CPU model, the cores this process may run on and the BLAS threads."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    return {"model": model, "cores": len(os.sched_getaffinity(0)), "blas_threads": int(threads)}


def cpu_plan():
    """The CPU-baseline table: one oracle draft pass (median of 3) for the
    smallest configuration (ctx 32, block 4), the short prompt (ctx 2432,
    block 8), the decode-loop shape (ctx 8192, block 8) and the quantized
    backbones (ctx 8192, block 4), the first two also on one thread, plus
    the short prompt's fusion and projection in full.  The oracle is the
    fp64 numpy one, as it stands; every matrix is decoded once before the
    timed calls.  Prints a markdown table and one JSON line."""
    import json as _json
    from threadpoolctl import threadpool_limits

    from block_draft_model_pass_amd import synth
    from oracle import dflash_oracle as O
    info = host_cpu()
    print(f"CPU: {info['model']}; {info['cores']} cores available, "
          f"BLAS threads {info['blas_threads']}", flush=True)
    rows = []

    def med(fn, n=3):
        ts = []
        for _ in range(n):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    def context(w, n):
        store = O.ContextStore()
        for s0 in range(0, n, 2048):
            taps = synth.make_taps(range(s0, min(n, s0 + 2048)))
            store.put(*O.project_ctx_kv(w, O.fuse_context(w, taps), s0), s0)
        return store

    def add(name, sec, nbytes=None, threads="all"):
        rec = {"config": name, "threads": threads, "seconds": round(sec, 3),
               "per_s": round(1.0 / sec, 3)}
        if nbytes:
            rec["GBs"] = round(nbytes / sec / 1e9, 2)
        rows.append(rec)
        print(_json.dumps(rec), flush=True)

    for fmt in ("bf16", "q8_0", "q4_0", "q5_0"):
        w = O.enable_cache(dict(synth.make_weights(fmt=fmt)))
        shapes = ((32, 4), (2432, 8), (8192, 8)) if fmt == "bf16" else ((8192, 4),)
        for n, b in shapes:
            store = context(w, n)
            ck, cv = store.window(n)
            anchor = synth.anchor_token(n)
            run = lambda: O.draft_block(w, ck, cv, n, anchor, synth.MASK_ID, b)  # noqa: E731
            run()  # decodes and caches every matrix
            add(f"draft ctx {n} block {b} {fmt}", med(run), pass_bytes(n, b, fmt))
            if fmt == "bf16" and n < 8192:
                with threadpool_limits(limits=1):
                    add(f"draft ctx {n} block {b} {fmt}", med(run), pass_bytes(n, b, fmt),
                        threads=1)
            if fmt == "bf16" and n == 2432:
                taps = synth.make_taps(range(n))
                ctx = O.fuse_context(w, taps)
                add("fusion 2432 x 12800 @ 12800 x 2560", med(lambda: O.fuse_context(w, taps), 1))
                add("K/V projection 2432 rows", med(lambda: O.project_ctx_kv(w, ctx, 0), 1))
        del w
    print("| measurement | threads | s | per s | GB/s |")
    print("|---|---|---:|---:|---:|")
    for r in rows:
        print(f"| {r['config']} | {r['threads']} | {r['seconds']} | {r['per_s']} | "
              f"{r.get('GBs', '')} |")
    print(_json.dumps({"cpu": info, "kind": "oracle (fp64 numpy)", "rows": rows}))


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the CPU-oracle baseline (0 = skip)")
    ap.add_argument("--reps", type=int, default=50, help="repeats of the event-timed kernels")
    ap.add_argument("--fusion-rows", type=int, default=32768,
                    help="rows of the timed context-fusion GEMM (0 = skip)")
    ap.add_argument("--cpu-plan", action="store_true",
                    help="only time the CPU oracle over the baseline plan's configurations "
                         "(no GPU) and print the table")
    ap.add_argument("--no-quant", action="store_true",
                    help="skip the Q8_0 / Q4_0 / Q5_0 backbone passes (ctx 8192, block 4)")
    args = ap.parse_args()
    if args.cpu_plan:
        cpu_plan()
        return
    if args.gpus != 1:
        print(f"bench.py: the draft pass runs on one GPU only (asked for --gpus {args.gpus}); "
              "there is no multi-GPU path (the pass's split of the LM-head vocabulary and "
              "of the KV heads over GPUs is not built).", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_draft_model_pass_amd import synth
    from block_draft_model_pass_amd.device import DeviceWeights, Drafter, KVRing, to_device

    torch.cuda.set_device(0)
    host_w = synth.make_weights()
    dw = DeviceWeights(host_w)
    kv = KVRing(synth.WINDOW, synth.WINDOW)
    dr = Drafter(dw, kv, max_rows=CTX)
    V = dw.vocab
    K = BLOCK - 1

    # Context 0..8191 and the taps of every position a job can commit.
    span = CTX + max(JOB_TOKENS, JOB_CYCLES * BLOCK) + BLOCK
    taps_all = to_device(synth.make_taps(range(span)))
    taps_ptr, tap_row_bytes = taps_all.data_ptr(), taps_all.stride(0) * taps_all.element_size()
    dr.commit(taps_all[:CTX], 0)
    n_pass = args.steps + args.warmup
    draws = [synth.target_draws(t, K) for t in range(n_pass)]
    match = torch.tensor(np.stack([d[0] for d in draws]), device="cuda")
    # int32 throughout: cand + 1 + r < 2 V < 2^31
    offset = torch.tensor(np.stack([d[1] for d in draws]) + 1, dtype=torch.int32, device="cuda")
    # targets per pass: K slots filled from the candidates each cycle, then the
    # stand-in target's continuation token
    tgt_all = torch.zeros((n_pass, K + 1), dtype=torch.int32, device="cuda")
    tgt_all[:, K] = torch.tensor([d[2] for d in draws], dtype=torch.int32, device="cuda")
    cand = torch.empty(K, dtype=torch.int32, device="cuda")
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def run_cycles(fused: bool):
        """W warm-up then K timed decode cycles; returns (seconds, accepted,
        offered).  Fused: one dflash_draft_block_commit per cycle commits the
        previous cycle's accepted cells and drafts the next block; otherwise
        draft, then the commit as its own fuse + project calls."""
        st = {"p": CTX, "anchor": synth.anchor_token(0), "job": 0, "acc": 0, "off": 0, "n": 0}

        def cycle(t):
            p = st["p"]
            if fused:
                n = st["n"]
                dr.draft_commit(taps_ptr + (p - n) * tap_row_bytes if n else None, n, p,
                                st["anchor"], BLOCK, cand=cand)
            else:
                dr.draft(p, st["anchor"], BLOCK, cand=cand)
            # stand-in target: the candidate where the draw matched, else another id
            tgt = tgt_all[t]
            torch.where(match[t], cand, torch.remainder(cand + offset[t], V), out=tgt[:K])
            dr.verify(cand, tgt, K, out=out)
            a, nxt = out.tolist()  # the cycle's one device->host read
            if fused:
                st["n"] = a + 1  # committed by the next cycle's pass
            else:
                dr.commit_ptr(taps_ptr + p * tap_row_bytes, a + 1, p)
            st["acc"] += a
            st["off"] += K
            st["p"], st["anchor"] = p + a + 1, nxt
            if st["p"] - CTX >= JOB_TOKENS:
                st["job"] += 1
                st["p"], st["anchor"], st["n"] = CTX, synth.anchor_token(st["job"]), 0

        for t in range(args.warmup):
            cycle(t)
        st["acc"] = st["off"] = 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(args.warmup, n_pass):
            cycle(t)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, st["acc"], st["off"]

    def run_device_cycles():
        """The fused cycle with its positions in device words: the pass reads
        {p, anchor, n_commit} and the verify advances them
        (dflash_draft_block_commit_dev, dflash_verify_greedy_advance), so no
        cycle reads from the device; a job restarts at position 8192 every
        JOB_CYCLES cycles by a device-to-device copy of its initial state.
        Returns (seconds, accepted, offered) over the timed cycles."""
        taps_ctx = taps_all[CTX:]
        jobs = (n_pass + JOB_CYCLES - 1) // JOB_CYCLES
        init = torch.tensor([[CTX, synth.anchor_token(j), 0] for j in range(jobs)],
                            dtype=torch.int64, device="cuda")
        dstate = torch.empty(3, dtype=torch.int64, device="cuda")
        outs = torch.empty((n_pass, 2), dtype=torch.int32, device="cuda")
        tgts = torch.zeros((n_pass, K + 1), dtype=torch.int32, device="cuda")
        tgts[:, K] = tgt_all[:, K]

        def cycle(t):
            if t % JOB_CYCLES == 0:
                dstate.copy_(init[t // JOB_CYCLES])
            dr.draft_commit_dev(taps_ctx, CTX, dstate, BLOCK, cand=cand)
            torch.where(match[t], cand, torch.remainder(cand + offset[t], V), out=tgts[t, :K])
            dr.verify_advance(cand, tgts[t], K, dstate, out=outs[t])

        for t in range(args.warmup):
            cycle(t)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(args.warmup, n_pass):
            cycle(t)
        torch.cuda.synchronize()
        dt_ = time.perf_counter() - t0
        a_ = outs[args.warmup:, 0].sum().item()
        st = torch.empty(1, dtype=torch.int32, device="cuda")
        dr.status(st)
        assert int(st.item()) == 0, "device-resident cycle: a pass reported a failure"
        return dt_, int(a_), K * args.steps

    def run_graph_cycles():
        """The device-resident cycle with each job of JOB_CYCLES cycles
        captured once as a HIP graph (the state reset, then every cycle's
        pass, stand-in target and verify) and replayed per job; between
        replays the host copies the next job's target draws into the graph's
        input buffers.  Returns (seconds, cycles) over the timed jobs."""
        taps_ctx = taps_all[CTX:]
        jobs = max(1, args.steps // JOB_CYCLES)
        init = torch.tensor([[CTX, synth.anchor_token(j), 0] for j in range(jobs + 1)],
                            dtype=torch.int64, device="cuda")
        s0 = torch.empty(3, dtype=torch.int64, device="cuda")
        dstate = torch.empty(3, dtype=torch.int64, device="cuda")
        m_job = torch.empty((JOB_CYCLES, K), dtype=match.dtype, device="cuda")
        o_job = torch.empty((JOB_CYCLES, K), dtype=torch.int32, device="cuda")
        t_job = torch.zeros((JOB_CYCLES, K + 1), dtype=torch.int32, device="cuda")
        o_out = torch.empty((JOB_CYCLES, 2), dtype=torch.int32, device="cuda")

        def load(j):  # job j's draws (cycles j*JOB_CYCLES ..., wrapping over the drawn ones)
            idx = torch.arange(j * JOB_CYCLES, (j + 1) * JOB_CYCLES, device="cuda") % n_pass
            m_job.copy_(match[idx])
            o_job.copy_(offset[idx])
            t_job[:, K] = tgt_all[idx, K]
            s0.copy_(init[j])

        load(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dstate.copy_(s0)
            for c in range(JOB_CYCLES):
                dr.draft_commit_dev(taps_ctx, CTX, dstate, BLOCK, cand=cand)
                torch.where(m_job[c], cand, torch.remainder(cand + o_job[c], V), out=t_job[c, :K])
                dr.verify_advance(cand, t_job[c], K, dstate, out=o_out[c])
        g.replay()  # warm-up job
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for j in range(1, jobs + 1):
            load(j)
            g.replay()
        torch.cuda.synchronize()
        dt_ = time.perf_counter() - t0
        st = torch.empty(1, dtype=torch.int32, device="cuda")
        dr.status(st)
        assert int(st.item()) == 0, "graph-replayed cycle: a pass reported a failure"
        del g
        return dt_, jobs * JOB_CYCLES

    dt_unfused, _, _ = run_cycles(False)
    dt_host, _, _ = run_cycles(True)
    dt, acc, off = run_device_cycles()
    dt_graph, n_graph = run_graph_cycles()
    value = args.steps / dt
    state = {"acc": acc, "off": off}

    # Draft pass alone, back to back at ctx 8192 (HIP events on the stream):
    # the median of 5 repeats of `reps` passes after 20 warm-up passes.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(20):
        dr.draft(CTX, 11, BLOCK, cand=cand)
    rep_ms = []
    for _ in range(5):
        ev[0].record()
        for _ in range(args.reps):
            dr.draft(CTX, 11, BLOCK, cand=cand)
        ev[1].record()
        torch.cuda.synchronize()
        rep_ms.append(ev[0].elapsed_time(ev[1]) / args.reps)
    draft_ms = float(np.median(rep_ms))
    draft_gbs = pass_bytes(CTX) / (draft_ms * 1e-3) / 1e9
    # The same pass with the confidence gate (softmax normaliser kept in the
    # LM-head sweep, floor 0.5): same weight bytes, a few exp per logit.
    g_cand = torch.empty(BLOCK - 1, dtype=torch.int32, device="cuda")
    g_conf = torch.empty(BLOCK - 1, dtype=torch.float32, device="cuda")
    g_keep = torch.empty(1, dtype=torch.int32, device="cuda")
    for _ in range(20):
        dr.draft_gated(CTX, 11, BLOCK, 0.5, cand=g_cand, conf=g_conf, n_keep=g_keep)
    g_ms = []
    for _ in range(5):
        ev[0].record()
        for _ in range(args.reps):
            dr.draft_gated(CTX, 11, BLOCK, 0.5, cand=g_cand, conf=g_conf, n_keep=g_keep)
        ev[1].record()
        torch.cuda.synchronize()
        g_ms.append(ev[0].elapsed_time(ev[1]) / args.reps)
    gated_ms = float(np.median(g_ms))

    # Standalone LM head + greedy argmax (the pass's largest single stream),
    # for reference beside the whole-pass kernel.
    z = torch.randn((K, synth.HIDDEN), device="cuda").to(torch.bfloat16).view(torch.int16)
    for _ in range(5):
        dr.lm_head_argmax(z, cand)
    ev[0].record()
    for _ in range(args.reps):
        dr.lm_head_argmax(z, cand)
    ev[1].record()
    torch.cuda.synchronize()
    lm_ms = ev[0].elapsed_time(ev[1]) / args.reps
    lm_gbs = lm_head_bytes() / (lm_ms * 1e-3) / 1e9

    def time_calls(fn, reps, warm=3):
        """Mean ms per call of `fn` over `reps` back-to-back calls after `warm`
        untimed ones (HIP events on the stream the calls run on)."""
        for _ in range(warm):
            fn()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    HT = synth.N_TAPS * synth.HIDDEN
    KVN = 2 * synth.N_LAYERS * synth.N_KV_HEADS * synth.HEAD_DIM  # Wk/Wv rows, all layers

    def gpu_taps(n, seed):
        gen = torch.Generator(device="cuda").manual_seed(seed)
        t = torch.randn((n, HT), generator=gen, device="cuda")
        return t.to(torch.bfloat16).view(torch.int16)

    # Long resident context: the 32768-row context fusion [n][12800] x
    # [12800][2560] bf16 on MFMA plus the RMSNorm epilogue (dflash_fuse_context),
    # the K/V projection of those rows into cells at positions
    # 229376..262143 (dflash_project_ctx_kv: [n][2560] x [2560][5120] GEMM, then
    # per-head norm, RoPE and the fp16 ring store), and the draft pass of a
    # block of 8 at 262144 over all 32768 resident cells.
    fusion = None
    long_ctx = None
    if args.fusion_rows > 0:
        nf = args.fusion_rows
        taps_f = gpu_taps(nf, 5)
        lring = KVRing(synth.WINDOW, synth.WINDOW)
        fdr = Drafter(dw, lring, max_rows=nf)
        ctx_f = fdr.fuse(taps_f)
        # the clock settles under sustained MFMA load during the warm-up calls
        f_ms = time_calls(lambda: fdr.fuse(taps_f, ctx_f), max(5, args.reps // 5))
        flops = 2.0 * nf * HT * synth.HIDDEN
        fusion = {"rows": nf, "shape": f"{nf}x{HT} @ {HT}x{synth.HIDDEN} bf16",
                  "ms": round(f_ms, 4), "TFLOPs": round(flops / (f_ms * 1e-3) / 1e12, 1),
                  "frac_bf16_mfma_peak": round(flops / (f_ms * 1e-3) / 2.5e15, 4),
                  "includes": "k_gemm_bf16_nt (bf16 rows + tile sums of squares) + k_rownorm_tiles; "
                              "k split in two + k_rownorm where that finishes sooner (dflash_fuse_context)"}
        if nf == synth.WINDOW:
            pos0 = 7 * synth.WINDOW  # 229376: the last 32768 positions before 262144
            p_ms = time_calls(lambda: fdr.project(ctx_f, pos0), max(5, args.reps // 5))
            p_flops = 2.0 * nf * synth.HIDDEN * KVN
            p = pos0 + nf
            l_ms = time_calls(lambda: fdr.draft(p, 11, BLOCK, cand=cand), args.reps, warm=5)
            l_bytes = pass_bytes(nf)
            long_ctx = {"cells": nf, "positions": [pos0, p - 1], "block_at": p,
                        "projection": {"shape": f"{nf}x{synth.HIDDEN} @ {synth.HIDDEN}x{KVN} bf16",
                                       "ms": round(p_ms, 4),
                                       "TFLOPs": round(p_flops / (p_ms * 1e-3) / 1e12, 1),
                                       "frac_bf16_mfma_peak": round(p_flops / (p_ms * 1e-3) / 2.5e15, 4),
                                       "includes": "k_rope_rows + k_gemm_bf16_nt writing the cells from its "
                                                   "epilogue (dflash_project_ctx_kv)"},
                        "draft": {"ms_per_pass": round(l_ms, 4), "passes_per_s": round(1e3 / l_ms, 2),
                                  "algorithmic_bytes": l_bytes,
                                  "achieved_GBs": round(l_bytes / (l_ms * 1e-3) / 1e9, 1),
                                  "frac_hbm_peak": round(l_bytes / (l_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
        del fdr, taps_f, ctx_f, lring
        torch.cuda.empty_cache()

    # Short prompt: fusion and K/V projection of a 2432-position prompt, then a
    # block of 8 drafted at 2432 over those cells.
    ns = 2432
    taps_s = gpu_taps(ns, 6)
    sdr = Drafter(dw, KVRing(2560, 2560), max_rows=ns)
    ctx_s = sdr.fuse(taps_s)
    s_f_ms = time_calls(lambda: sdr.fuse(taps_s, ctx_s), args.reps // 5 or 1)
    s_p_ms = time_calls(lambda: sdr.project(ctx_s, 0), args.reps // 5 or 1)
    s_d_ms = time_calls(lambda: sdr.draft(ns, 11, BLOCK, cand=cand), args.reps, warm=5)
    s_fl, s_pl, s_bytes = 2.0 * ns * HT * synth.HIDDEN, 2.0 * ns * synth.HIDDEN * KVN, pass_bytes(ns)
    short = {"ctx": ns, "block": BLOCK,
             "fusion": {"ms": round(s_f_ms, 4), "TFLOPs": round(s_fl / (s_f_ms * 1e-3) / 1e12, 1),
                        "frac_bf16_mfma_peak": round(s_fl / (s_f_ms * 1e-3) / 2.5e15, 4)},
             "projection": {"ms": round(s_p_ms, 4), "TFLOPs": round(s_pl / (s_p_ms * 1e-3) / 1e12, 1),
                            "frac_bf16_mfma_peak": round(s_pl / (s_p_ms * 1e-3) / 2.5e15, 4)},
             "draft": {"ms_per_pass": round(s_d_ms, 4), "passes_per_s": round(1e3 / s_d_ms, 2),
                       "algorithmic_bytes": s_bytes,
                       "achieved_GBs": round(s_bytes / (s_d_ms * 1e-3) / 1e9, 1),
                       "frac_hbm_peak": round(s_bytes / (s_d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
    del sdr, taps_s, ctx_s
    torch.cuda.empty_cache()

    # Quantized backbone (Q8_0 / Q4_0 / Q5_0 layer matrices, bf16 LM head): draft
    # passes at ctx 8192, block 4, on a context projected by those weights.
    # Also the Q8_0 shared LM head: bf16 backbone at blocks 8 and 4, and with
    # a Q8_0 backbone at block 4 (every streamed matrix in Q8_0).
    quant, q8_lm = {}, {}
    if not args.no_quant:
        runs = (("q8_0", "bf16", (4,)), ("q4_0", "bf16", (4,)), ("q5_0", "bf16", (4,)),
                ("q8_0", "q8_0", (4,)), ("bf16", "q8_0", (8, 4)))
        for fmt, lmf, blocks in runs:
            qw = DeviceWeights(synth.make_weights(fmt=fmt, lm_fmt=lmf))
            qkv_ring = KVRing(synth.WINDOW, synth.WINDOW)
            qdr = Drafter(qw, qkv_ring, max_rows=2048)
            for s0 in range(0, CTX, 2048):
                qdr.commit(to_device(synth.make_taps(range(s0, s0 + 2048))), s0)
            for qb in blocks:
                for _ in range(5):
                    qdr.draft(CTX, 11, qb, cand=cand)
                ev[0].record()
                for _ in range(args.reps):
                    qdr.draft(CTX, 11, qb, cand=cand)
                ev[1].record()
                torch.cuda.synchronize()
                q_ms = ev[0].elapsed_time(ev[1]) / args.reps
                q_bytes = pass_bytes(CTX, qb, fmt, lmf)
                q_gbs = q_bytes / (q_ms * 1e-3) / 1e9
                rec = {"ctx": CTX, "block": qb, "backbone": fmt, "lm_head": lmf,
                       "ms_per_pass": round(q_ms, 4),
                       "passes_per_s": round(1e3 / q_ms, 2), "algorithmic_bytes": q_bytes,
                       "achieved_GBs": round(q_gbs, 1),
                       "frac_hbm_peak": round(q_gbs / HBM_PEAK_GBS, 4)}
                if fmt == "bf16":
                    q8_lm[f"block{qb}"] = rec
                else:
                    quant[fmt if lmf == "bf16" else f"{fmt}+{lmf}_lm_head"] = rec
            del qdr, qkv_ring, qw
            torch.cuda.empty_cache()

    # Attainable rates of this device, for reference beside the kernels: a
    # 1 GiB device-to-device copy (bytes read + written per second) and the
    # vendor BLAS (torch.mm) on the context-fusion shape.
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    c_ms = time_calls(lambda: dst.copy_(src), 10)
    copy_gbs = 2 * src.numel() * 4 / (c_ms * 1e-3) / 1e9
    del src, dst
    attainable = {"copy_1GiB": {"ms": round(c_ms, 4), "GBs_read_plus_write": round(copy_gbs, 1),
                                "frac_hbm_peak": round(copy_gbs / HBM_PEAK_GBS, 4)}}
    if args.fusion_rows > 0:
        nf = args.fusion_rows
        gen = torch.Generator(device="cuda").manual_seed(7)
        a_ = torch.randn((nf, HT), generator=gen, device="cuda").to(torch.bfloat16)
        b_ = torch.randn((HT, synth.HIDDEN), generator=gen, device="cuda").to(torch.bfloat16)
        v_ms = time_calls(lambda: torch.mm(a_, b_), max(5, args.reps // 5))
        v_fl = 2.0 * nf * HT * synth.HIDDEN
        attainable["vendor_bf16_gemm"] = {"shape": f"{nf}x{HT} @ {HT}x{synth.HIDDEN}",
                                          "ms": round(v_ms, 4),
                                          "TFLOPs": round(v_fl / (v_ms * 1e-3) / 1e12, 1),
                                          "frac_bf16_mfma_peak": round(v_fl / (v_ms * 1e-3) / 2.5e15, 4),
                                          "note": "torch.mm (bf16 output, no norm)"}
        del a_, b_
        torch.cuda.empty_cache()

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(host_w, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "passes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * dt / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "DFlash decode cycle: 8192 resident context cells, block 8 "
                               "(anchor + 7 masks), greedy verify vs Bernoulli(0.75) stand-in "
                               "target; the accepted cells are committed by the next cycle's "
                               "pass; positions in device words advanced by the verify "
                               "(dflash_draft_block_commit_dev, dflash_verify_greedy_advance), "
                               f"jobs of {JOB_CYCLES} cycles from position 8192",
                   "ctx": CTX, "block": BLOCK, "vocab": V, "backbone": "bf16"},
        "decode_cycle_host_positions": {
            "ms_per_cycle": round(1e3 * dt_host / args.steps, 4),
            "cycles_per_s": round(args.steps / dt_host, 3),
            "note": "the same fused cycle with the positions as host arguments "
                    "(dflash_draft_block_commit): one device-to-host read of (accepted, "
                    "next) per cycle; 96-token jobs"},
        "decode_cycle_graph": {"ms_per_cycle": round(1e3 * dt_graph / n_graph, 4),
                               "cycles_per_s": round(n_graph / dt_graph, 3),
                               "cycles": n_graph,
                               "note": f"the device-resident cycle with each job of {JOB_CYCLES} "
                                       "cycles captured once as a HIP graph and replayed; the "
                                       "next job's draws are copied in between replays"},
        "decode_cycle_unfused": {"ms_per_cycle": round(1e3 * dt_unfused / args.steps, 4),
                                 "cycles_per_s": round(args.steps / dt_unfused, 3),
                                 "note": "draft, verify, then the commit as separate fuse + "
                                         "project calls"},
        "draft_only": {"ms_per_pass": round(draft_ms, 4),
                       "ms_range_of_5_repeats": [round(min(rep_ms), 4), round(max(rep_ms), 4)],
                       "passes_per_s": round(1e3 / draft_ms, 2),
                       "algorithmic_bytes": pass_bytes(CTX),
                       "achieved_GBs": round(draft_gbs, 1),
                       "frac_hbm_peak": round(draft_gbs / HBM_PEAK_GBS, 4)},
        # The draft pass is one persistent kernel (k_draft_pass, after the tiny
        # k_pass_init); events bracket both on the stream they run on.
        "roofline": {"kernel": "k_draft_pass (dflash_draft_block, ctx 8192, block 8)",
                     "bound": "hbm", "achieved": round(draft_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(draft_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(), "launch_ms": round(draft_ms, 4),
                     "bytes_per_launch": pass_bytes(CTX)},
        "gated_draft": {"entry": "dflash_draft_block_gated (min_p 0.5)",
                        "ms_per_pass": round(gated_ms, 4),
                        "ms_range_of_5_repeats": [round(min(g_ms), 4), round(max(g_ms), 4)],
                        "passes_per_s": round(1e3 / gated_ms, 2),
                        "overhead_vs_plain": round(gated_ms / draft_ms - 1.0, 4)},
        "lm_head_standalone": {"kernel": "k_lmhead_bf16 + k_argmax_reduce (dflash_lm_head_argmax)",
                               "ms": round(lm_ms, 4), "bytes": lm_head_bytes(),
                               "achieved_GBs": round(lm_gbs, 1),
                               "frac_hbm_peak": round(lm_gbs / HBM_PEAK_GBS, 4)},
        "fusion_gemm": fusion,
        "long_context": long_ctx,
        "short_prompt": short,
        "attainable": attainable,
        "quantized_backbone": quant or None,
        "q8_0_lm_head": q8_lm or None,
        "accepted_offered": [state["acc"], state["off"]],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
