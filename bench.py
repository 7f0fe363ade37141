"""Decode-step benchmark: one attention layer's absorbed-MLA decode on one GPU.

A step is the whole hot path on one batch: rope_relocate_q (per distinct
segment shift) and mla_absorb_q (one mla_prepare_q launch) ->
mla_decode_splitkv -> mla_combine_lse -> mla_out_uv, on seeded synthetic
inputs already resident in HBM.  Prints one
JSON line with decode tokens/s, the decode kernel's achieved HBM GB/s against
the MI355X roofline, and the fp64 CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3]

The default workload is the largest single-GPU configuration: the
DeepSeek-V3-style batch (B=64, H=128, T_b ~ U[1024, 32768], 64-row pages).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode tokens/s + achieved HBM GB/s & % roofline (latent-cache attention)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
MALL_BYTES = 256 << 20          # Infinity Cache: rotate caches so every step reads HBM
DECODE_SRCS = [os.path.join(ROOT, "mla_latent_cache_amd", "csrc", f)
               for f in ("mla_decode_bf16.hip", "mla_decode_rows.hip", "mla_decode_tile.h", "mla_common.h",
                         "mla_kernels.h")]
SEEDS = {"toy": 0, "small": 1, "dsv3": 2, "long": 3, "merge": 4, "prefill": 5, "qknorm": 6, "int8": 7, "int4": 8,
         "qknorm_dsv3": 9}


def _rows(x):
    return [int(s.seq_lens.sum()) for s in x.segments]


def algorithmic(x):
    """Decode-kernel algorithmic bytes and FLOPs per launch: every stored row
    [c_t | kr_t] read once (1152 B in bf16), and per visible (row, query row)
    pair 2 * (576 + 512) FLOPs (scores over [c | kr], weighted sum over c).
    A causal segment shows query s of s_q the rows t <= T - s_q + s.  With
    QK-Norm each row also brings its 4-byte inverse key RMS; an int8 cache row
    is d_c one-byte codes, the 16-bit rotary key and a 4-byte scale (644 B);
    an int4 row is (d_c + d_rope) / 2 bytes of codes and two 4-byte scales
    (296 B)."""
    sp = x.spec
    el = x.segments[0].cache.element_size()
    if sp.quant == "int8":
        row = sp.d_c + 2 * sp.d_rope + 4
    elif sp.quant == "int4":
        row = (sp.d_c + sp.d_rope) // 2 + 8
    else:
        row = sp.row_width * el + (4 if sp.qk_norm else 0)
    nbytes = sum(r * row for r in _rows(x))
    flops = 0
    for s in x.segments:
        for T in s.seq_lens.tolist():
            pairs = sum(max(0, min(T, T - sp.s_q + q + 1)) for q in range(sp.s_q)) if s.causal else T * sp.s_q
            flops += 2 * pairs * s.head_count * (sp.row_width + sp.d_c)
    return nbytes, flops


def ops_cache_dt(step) -> int:
    from mla_latent_cache_amd import ops
    return ops._cache_dt(step.segments[0].cache, step.segments[0].row_scale)


def decode_kernel_name(x) -> str:
    """The decode kernel a workload's launches run (the routing of
    mla_decode_splitkv; 16-bit and low-bit caches write bf16 partials)."""
    sp = x.spec
    rows = [sp.s_q * (s.head_count or sp.heads) for s in x.segments]
    if sp.dtype != "bf16":
        return "decode_f32_kernel"
    if sp.quant in ("int4", "int8"):
        qm = 1 if sp.quant == "int4" else 2
        return f"decode_rows_kernel<1, {qm}, true> ({sp.quant} rows, 64-row groups)"
    if len(rows) == 1 and rows[0] <= 32:
        return "decode_bf16_kernel"
    rb = 1 if max(rows) <= 64 else 2
    qkn = ", QK-Norm row factors" if sp.qk_norm else ""
    return f"decode_rows_kernel<{rb}, 0, true> ({64 * rb}-row groups{qkn})"


def kernel_hash() -> str:
    """Hash of the code of the decode kernels' sources and the headers they
    include (the files that exist): comments removed and whitespace runs
    folded, so that an edit of the comments keeps the counters valid."""
    h = hashlib.sha256()
    for p in DECODE_SRCS:
        if os.path.exists(p):
            with open(p, encoding="utf-8") as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes of one step's decode work (every decode dispatch of a step,
    summed: a step over several segments may launch more than one) from the
    committed counter summary, or None when there is none or the decode
    sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_val = re.search(r"hbm_bytes_per_step:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_val or m_hash.group(1) != kernel_hash():
        return None
    return float(m_val.group(1))


def cpu_baseline(x, budget_s: float):
    """Time the oracle as it stands on a bounded sample of the same inputs:
    whole requests (all heads) in order until the budget is spent; for very
    long requests, chunks of heads.  Reported in query tokens/s."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle.mla_direct as O
    import oracle.mla_quant as Q

    def f64(t):
        return t.to(torch.float64).numpy()

    sp = x.spec

    def rows(s, b):  # as attention reads them (low-bit cache: the oracle's quantize/dequantize)
        if sp.quant == "int8":
            return Q.quantized_rows(s.rows(b).float().numpy(), sp.d_c)
        if sp.quant == "int4":
            return Q.quantized_rows_i4(s.rows(b).float().numpy(), sp.d_c)
        return f64(s.rows(b))

    segs = [O.OracleSegment(rows=(lambda b, s=s: rows(s, b)), shift=s.shift.tolist(),
                            head_begin=s.head_begin, head_count=s.head_count, causal=s.causal)
            for s in x.segments]
    q_nope, q_pe, w_uk, w_uv = f64(x.q_nope), f64(x.q_pe), f64(x.w_uk), f64(x.w_uv)
    q_pos = x.q_pos.numpy()
    qk = O.QKNorm(f64(x.g_q), f64(x.g_k), sp.qk_eps) if x.g_q is not None else None
    rows_per_req = max(_rows(x)) / sp.batch
    hchunk = sp.heads if rows_per_req * sp.heads <= 64 * 4096 else max(1, (64 * 4096) // int(rows_per_req) or 1)
    done_pairs = 0
    t0 = time.perf_counter()
    b = 0
    while True:
        for h0 in range(0, sp.heads, hchunk):
            hs = list(range(h0, min(sp.heads, h0 + hchunk)))
            O.direct_mla_decode(q_nope, q_pe, q_pos, w_uk, w_uv, segs, x.scale, x.rope_base, sp.s_q,
                                requests=[b % sp.batch], heads=hs, qk_norm=qk)
            done_pairs += len(hs)
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
        b += 1
    el = time.perf_counter() - t0
    tokens = done_pairs / sp.heads * sp.s_q
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {"value": tokens / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done_pairs} (request, head) pairs = {tokens:.3g} query tokens of the same seeded "
                      f"workload, fp64 direct form, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3", choices=["small", "dsv3", "long", "merge", "toy", "prefill", "qknorm", "int8", "int4",
                                                               "qknorm_dsv3"])
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--n-wg", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--detail", action="store_true", help="also time each call separately")
    ap.add_argument("--eager", action="store_true", help="host launches instead of a HIP graph")
    ap.add_argument("--no-fuse-post", action="store_true",
                    help="merge and U_V as two calls even for few query tokens")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="before the timed region, run one plain device copy of this many bytes (fp32 "
                         "elementwise, read N and write N) whose HBM counters calibrate the decode kernel's")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the decode path has no multi-GPU mode in this library "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import mla_inputs as M
    from mla_latent_cache_amd import load
    from mla_latent_cache_amd.step import DecodeStep, StepSegment, run_calls, step_from_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    load()
    torch.cuda.set_device(0)
    seed = SEEDS[args.workload] if args.seed is None else args.seed
    x = M.make(args.workload, seed)
    sp = x.spec

    # Cache copies: enough that the rotated set exceeds twice the 256 MiB
    # Infinity Cache, so every step streams its cache from HBM.
    nbytes, flops = algorithmic(x)
    # (at most 64 copies: a cache of a few KiB, the toy, stays cached anyway)
    n_copies = min(64, max(1, math.ceil(2 * MALL_BYTES / max(1, nbytes))))
    fuse = False if args.no_fuse_post else None
    base = step_from_inputs(x, n_wg=args.n_wg, fuse_post=fuse)
    step_fused = base.fuse_post
    steps = [base]
    # every copy runs the same variant as the base step (QK-Norm factors of its
    # own cache, an int8 cache quantized from its own bf16 rows)
    qk = (base.g_q, base.g_k, base.qk_eps) if base.qk_norm else None
    for _ in range(n_copies - 1):
        segs = []
        for bs, s in zip(base.segments, x.segments):
            shift_tok = x.token_shift(s)
            cache = s.cache.to(bs.cache.device) if sp.quant else bs.cache.clone()
            segs.append(StepSegment(cache=cache, seq_lens=bs.seq_lens, seq_lens_host=s.seq_lens.tolist(),
                                    shift=shift_tok.to(bs.cache.device), shift_host=shift_tok.tolist(),
                                    block_table=bs.block_table, head_begin=bs.head_begin,
                                    head_count=bs.head_count, causal=bs.causal))
        steps.append(DecodeStep(base.q_nope, base.q_pe, base.q_pos, base.w_uk, base.w_uv, segs, sp.batch, sp.s_q,
                                x.scale, x.rope_base, n_wg=args.n_wg, n_split=base.n_split, fuse_post=fuse,
                                qk_norm=qk, quant=sp.quant))
    assert all(st.qk_norm == base.qk_norm and ops_cache_dt(st) == ops_cache_dt(base) for st in steps)
    # Launch path.  Graph mode (default): the step is captured into a HIP
    # graph of U consecutive steps (cycling the cache copies) and the timed
    # region replays it, so small workloads are bound by the GPU rather than
    # by five host launches per step.  The decode kernel's duration is then
    # timed, right after the timed region, by HIP events around a graph of U
    # back-to-back decode launches (so it includes the dispatch gap between
    # kernels; HIP does not allow timing events inside a captured graph).
    # Eager mode (--eager, or if capture fails): host launches, with events
    # around every decode launch inside the timed region.
    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    launch = "eager" if args.eager else "graph"
    dec_us = None
    if launch == "graph":
        try:
            cap = torch.cuda.Stream()
            bound_cap = [st.bind(cap) for st in steps]
            U = n_copies * max(1, math.ceil(8 / n_copies))

            def build_graph(n_steps, parts=("pre", "dec", "post")):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    for k in range(n_steps):
                        pre, dec, post = bound_cap[k % n_copies]
                        for name, calls in zip(("pre", "dec", "post"), (pre, dec, post)):
                            if name in parts:
                                run_calls(calls)
                return g

            g_full = build_graph(U)
            rem = args.steps % U
            g_rem = build_graph(rem) if rem else None
            g_dec = build_graph(U, parts=("dec",))
            for _ in range(max(1, math.ceil(args.warmup / U))):
                g_full.replay()
            g_dec.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps // U):
                g_full.replay()
            if g_rem is not None:
                g_rem.replay()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(1, math.ceil(args.steps / U))
            e0.record()
            for _ in range(reps):
                g_dec.replay()
            e1.record()
            torch.cuda.synchronize()
            dec_us = 1000.0 * e0.elapsed_time(e1) / (reps * U)
        except Exception as e:  # noqa: BLE001 - fall back to host launches, and say so
            print(f"graph capture unavailable ({type(e).__name__}: {e}); timing host launches", file=sys.stderr)
            launch = "eager"
    stream = torch.cuda.current_stream()
    bound = [st.bind(stream) for st in steps]

    def one(i, ev=None):
        pre, dec, post = bound[i % n_copies]
        run_calls(pre)
        if ev is not None:
            ev[0].record(stream)
        run_calls(dec)
        if ev is not None:
            ev[1].record(stream)
        run_calls(post)

    if launch == "eager":
        for i in range(args.warmup):
            one(i)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            one(i, evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        dec_ms = [a.elapsed_time(b) for a, b in evs]
        dec_us = 1000.0 * sum(dec_ms) / len(dec_ms)
    elapsed = t1 - t0

    detail = None
    if args.detail:
        # each call alone, back to back on the stream (host launches)
        detail = {}
        reps = 50
        names = ["prepare", "decode"] + (["combine_out_uv"] if step_fused else ["combine", "out_uv"])
        for nm in names:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for j in range(reps):
                pj, dj, qj = bound[j % n_copies]
                g = {"prepare": pj, "decode": dj, "combine": qj[:1], "out_uv": qj[1:], "combine_out_uv": qj}[nm]
                run_calls(g)
            e1.record(stream)
            torch.cuda.synchronize()
            detail[nm + "_us"] = round(1000.0 * e0.elapsed_time(e1) / reps, 3)

    n_tok = sp.n_tok
    value = n_tok * args.steps / elapsed
    achieved = nbytes / (dec_us * 1e-6) / 1e9
    tflops = flops / (dec_us * 1e-6) / 1e12
    # bound: HBM unless the arithmetic intensity exceeds the ridge of the bf16
    # MFMA and HBM peaks (the prefill chunk)
    mfma_bound = flops / max(1, nbytes) > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    traffic = traffic_from_profile(args.workload)
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1000.0 * elapsed / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sp.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": sp.description, "name": sp.name, "batch": sp.batch, "heads": sp.heads,
                   "s_q": sp.s_q, "d_c": sp.d_c, "d_rope": sp.d_rope, "d_nope": sp.d_nope, "d_v": sp.d_v,
                   "cache_rows": sum(_rows(x)), "seed": seed, "cache_copies_rotated": n_copies,
                   "parallelism": "single GPU", "launch": launch,
                   "post": "combine_out_uv" if step_fused else "combine_lse + out_uv"},
        "roofline": dict(
            ({"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
              "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic, "hbm_gbs": round(achieved, 2)}
             if mfma_bound else
             {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
              "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}),
            kernel=f"mla_decode_splitkv ({decode_kernel_name(x)})", decode_us=round(dec_us, 3),
            algorithmic_bytes=nbytes, algorithmic_flops=flops, tflops=round(tflops, 2),
            mfma_frac=round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)),
        "cpu_baseline": None,
    }
    if detail:
        res["detail"] = detail
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
