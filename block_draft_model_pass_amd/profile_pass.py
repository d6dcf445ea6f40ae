"""Profiling driver: draft passes at ctx 8192 for rocprofv3 runs.

Builds the synthetic drafter (bf16 by default), commits context positions
0..8191, then runs `--passes` draft passes of `--block` rows at position 8192
back to back (or, with `--fuse-rows n`, `--passes` context fusions of n
rows; with `--project-rows n`, `--passes` K/V projections of n fused rows
into a 32768-cell ring at positions 229376..).  With `--copy-mib M` it first copies an M MiB device buffer `--copies`
times (a plain copy kernel of known size, whose HBM counters calibrate those
of the pass kernel).  Prints one line per step it finishes.

    python -m block_draft_model_pass_amd.profile_pass --passes 20
"""
from __future__ import annotations

import argparse
import sys


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--passes", type=int, default=20)
    ap.add_argument("--block", type=int, default=8)
    ap.add_argument("--ctx", type=int, default=8192)
    ap.add_argument("--fmt", default="bf16", choices=["bf16", "q8_0", "q4_0", "q5_0"])
    ap.add_argument("--gated", type=float, default=None, metavar="MIN_P",
                    help="draft with the confidence gate at this floor "
                         "(dflash_draft_block_gated)")
    ap.add_argument("--commit", type=int, default=0, metavar="N",
                    help="fused draft-commit passes: each commits the N positions "
                         "before ctx and drafts at ctx (dflash_draft_block_commit)")
    ap.add_argument("--copy-mib", type=int, default=0)
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--fuse-rows", type=int, default=0,
                    help="instead of draft passes: context fusion of this many rows "
                         "(the bf16 GEMM + RMSNorm), --passes times")
    ap.add_argument("--project-rows", type=int, default=0,
                    help="instead of draft passes: K/V projection of this many rows "
                         "(the bf16 GEMM + per-head norm / RoPE / ring store), --passes times")
    args = ap.parse_args(argv)

    import torch

    from block_draft_model_pass_amd import synth
    from block_draft_model_pass_amd.device import DeviceWeights, Drafter, KVRing, to_device

    torch.cuda.set_device(0)
    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.copies):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {args.copy_mib} MiB x {args.copies}", flush=True)
        del src, dst
    dw = DeviceWeights(synth.make_weights(fmt=args.fmt))
    if args.fuse_rows > 0:
        nf = args.fuse_rows
        gen = torch.Generator(device="cuda").manual_seed(5)
        taps = torch.randn((nf, synth.N_TAPS * synth.HIDDEN), generator=gen, device="cuda")
        taps = taps.to(torch.bfloat16).view(torch.int16)
        fdr = Drafter(dw, KVRing(256), max_rows=nf)
        ctx = fdr.fuse(taps)
        for _ in range(args.passes):
            fdr.fuse(taps, ctx)
        torch.cuda.synchronize()
        print(f"{args.passes} fusions of {nf} rows done", flush=True)
        return 0
    if args.project_rows > 0:
        nr = args.project_rows
        gen = torch.Generator(device="cuda").manual_seed(5)
        ctx = torch.randn((nr, synth.HIDDEN), generator=gen, device="cuda")
        ctx = ctx.to(torch.bfloat16).view(torch.int16)
        pdr = Drafter(dw, KVRing(synth.WINDOW, synth.WINDOW), max_rows=nr)
        for _ in range(args.passes):
            pdr.project(ctx, 7 * synth.WINDOW)
        torch.cuda.synchronize()
        print(f"{args.passes} projections of {nr} rows done", flush=True)
        return 0
    dr = Drafter(dw, KVRing(synth.WINDOW, synth.WINDOW), max_rows=2048)
    nc = args.commit
    for s0 in range(0, args.ctx - nc, 2048):
        dr.commit(to_device(synth.make_taps(range(s0, min(args.ctx - nc, s0 + 2048)))), s0)
    ctaps = to_device(synth.make_taps(range(args.ctx - nc, args.ctx))) if nc else None
    torch.cuda.synchronize()
    print(f"context 0..{args.ctx - nc - 1} committed ({args.fmt})", flush=True)
    cand = torch.empty(8, dtype=torch.int32, device="cuda")
    conf = torch.empty(8, dtype=torch.float32, device="cuda")
    keep = torch.empty(1, dtype=torch.int32, device="cuda")
    for i in range(args.passes):
        if nc:  # the same nc cells rewritten every pass
            dr.draft_commit(ctaps.data_ptr(), nc, args.ctx, 11, args.block, cand=cand)
        elif args.gated is None:
            dr.draft(args.ctx, 11, args.block, cand=cand)
        else:
            dr.draft_gated(args.ctx, 11, args.block, args.gated, cand=cand[:args.block - 1],
                           conf=conf[:args.block - 1], n_keep=keep)
    torch.cuda.synchronize()
    gate = "" if args.gated is None else f", gated at min_p {args.gated}"
    gate += f", committing {nc} cells each" if nc else ""
    print(f"{args.passes} draft passes done, block {args.block}{gate}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
