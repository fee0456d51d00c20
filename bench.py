"""Benchmark: FP8 paged GQA decode on one MI355X.

One step = one decode call (pa_fp8_decode: every step of the path, through
the C ABI) over one batch of synthetic input already resident in HBM.  The
workload is the GLM-4.5-shaped decode (B=32, nq=96, nkv=8, D=128, block 128,
lengths U[1024, 8192], s2_tile 512).  Timed steps rotate over several
independent input sets (>= 1 GB together) so the 256 MB Infinity Cache
cannot serve them; a warm-cache figure (one set repeated) is printed too.

Prints ONE JSON line.  `value` is achieved GB/s of algorithmic bytes (K, V,
k_scale of every valid token and KV head, v_scale, Q, q_scale, output, the
table entries and lengths) per decode call.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "fp8_paged_kv_amd", "csrc", "pa_fp8_decode_rows.hip")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "decode_rows_kernel_glm45_b32_pmc.md")


def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="workload id (1-3 GQA, 4 MLA)")
    ap.add_argument("--op", choices=["decode", "scatter", "epilog", "ceiling", "fp8-mfma", "phases", "valu-rates",
                                     "prefill", "lds-patterns"],
                    default="decode",
                    help="scatter: the FP8 KV-cache writer filling config 1's pool (prefill-sized write); "
                         "epilog: KvCompressEpilog mode 1 on 131072 MLA-latent rows; "
                         "ceiling: read-only probes of config 1's paged access pattern and of a contiguous "
                         "buffer, beside the decode; valu-rates: issue rate of the FP8 dequantisation "
                         "instructions; prefill: the causal prefill chunk alone; lds-patterns: LDS read rate "
                         "of lane address patterns")
    ap.add_argument("--no-secondary", action="store_true",
                    help="headline only: skip the other workloads' entries")
    ap.add_argument("--secondary-steps", type=int, default=50)
    ap.add_argument("--splits", type=int, default=0, help="0 = library's choice")
    ap.add_argument("--causal", action="store_true",
                    help="GQA: causal multi-token decode (position s of s1 sees the first seq - s1 + 1 + s tokens)")
    ap.add_argument("--kv-split", action="store_true",
                    help="config 4: the MLA cache as three tensors (codes, rope, scales) instead of 672-byte rows")
    ap.add_argument("--rotate", type=int, default=3, help="independent input sets cycled by the timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-target-s", type=float, default=15.0, help="wall seconds budget of the oracle sample")
    ap.add_argument("--pmc-mode", action="store_true",
                    help="short fixed run for counter collection: decode calls plus a plain copy of known size")
    ap.add_argument("--sweep-splits", type=str, default="", help="comma list; prints one line per split count")
    return ap.parse_args()


def make_sets(cfg, n, device="cuda"):
    from fp8_paged_kv_amd import synth
    first = synth.make_gqa_inputs(cfg, device=device)
    seqs = first["kv_act_seqs"].cpu().tolist()
    sets = [first]
    for i in range(1, n):
        sets.append(synth.make_gqa_inputs(cfg, device=device, seed=1000 + 17 * i + cfg.seed, seq_lens=seqs))
    return sets, seqs


def _timed(call, steps, warmup, sample=100):
    """Warm-up, then exactly `steps` calls between two synchronisations: wall
    clock and two HIP events on the launch stream bracket them (no per-call
    events inside, they would add a barrier between the kernels of
    consecutive calls).  A separate, untimed pass with one event pair per call
    gives the per-call distribution.  Returns (wall s, region ms per call,
    sorted per-call ms)."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        call(i, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        call(i, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region = e0.elapsed_time(e1) / steps
    n = max(1, min(steps, sample))
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for i in range(n):
        starts[i].record(stream)
        call(i, stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    return wall, region, sorted(a.elapsed_time(b) for a, b in zip(starts, ends))


def time_calls(binding, sets, steps, warmup, splits, out, ws):
    def call(i, stream):
        binding.decode_inputs(sets[i % len(sets)], num_splits=splits, out=out, workspace=ws, stream=stream)
    return _timed(call, steps, warmup)


def cpu_baseline(cfg, host, seqs, target_s):
    """The oracle as it stands, on the first sequences of the same workload
    (``host``: the first timed input set, copied to the host)."""
    from fp8_paged_kv_amd import synth
    from oracle import oracle
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count() or 1
    threads = max(1, min(threads, 16))          # one GPU's share of the host
    # calibrate on one sequence, then size the sample to the time budget
    t0 = time.perf_counter()
    oracle.gqa_decode(host, b_range=(0, 1), threads=1)
    one = time.perf_counter() - t0
    per_tok = one / max(1, seqs[0])
    nb, acc = 0, 0.0
    for s in seqs:
        if nb > 0 and acc + per_tok * s / threads > target_s:
            break
        acc += per_tok * s / threads
        nb += 1
    used = min(threads, nb)
    t0 = time.perf_counter()
    oracle.gqa_decode(host, b_range=(0, nb), threads=used)
    dt = time.perf_counter() - t0
    sub = synth.GqaConfig(**{**cfg.__dict__, "B": nb})
    sample_bytes = synth.gqa_algorithmic_bytes(sub, seqs[:nb])
    one_bytes = synth.gqa_algorithmic_bytes(synth.GqaConfig(**{**cfg.__dict__, "B": 1}), seqs[:1])
    full_tokens = sum(seqs)
    return {"value": round(sample_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"sequences 0..{nb - 1} of {cfg.B} ({sum(seqs[:nb])} of {full_tokens} tokens, all "
                      f"{cfg.nq} query heads), FP64 C oracle, {dt:.2f} s wall on {used} threads",
            "calls_per_s_equiv": round((sum(seqs[:nb]) / full_tokens) / dt, 6),
            "single_thread": {"value": round(one_bytes / one / 1e9, 4), "unit": "GB/s",
                              "sample": f"sequence 0 ({seqs[0]} tokens, all {cfg.nq} query heads), 1 thread, "
                                        f"{one:.2f} s wall"}}


def pmc_traffic():
    """Counter-measured HBM bytes per decode launch, if the summary matches this kernel."""
    if not os.path.exists(PMC_SUMMARY):
        return None, "no counter summary"
    text = open(PMC_SUMMARY).read()
    m = re.search(r"kernel_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t:
        return None, "summary incomplete"
    if m.group(1) != kernel_hash():
        return None, "kernel changed since the counters were taken"
    return float(t.group(1)), "ok"


def main():
    args = parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 (no multi-GPU path)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from fp8_paged_kv_amd import binding, synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    binding.lib()
    if args.op == "scatter":
        return run_scatter(args)
    if args.op == "epilog":
        return run_epilog(args)
    if args.op == "ceiling":
        return run_ceiling(args)
    if args.op == "fp8-mfma":
        return run_fp8_mfma(args)
    if args.op == "phases":
        return run_phases(args)
    if args.op == "valu-rates":
        return run_valu_rates(args)
    if args.op == "lds-patterns":
        return run_lds_patterns(args)
    if args.op == "prefill":
        print(json.dumps(measure_gqa(None, True, args.steps, args.warmup, max(1, args.rotate), cfg=prefill_config())),
              flush=True)
        return
    if args.config == 4:
        return run_mla(args)
    cfg = synth.CONFIGS[args.config]
    sets, seqs = make_sets(cfg, max(1, args.rotate))
    if args.causal:
        if args.splits:
            sys.exit("--causal runs on the whole-row path (--splits 0)")
        for st in sets:
            st["causal"] = True
    nbytes = synth.gqa_algorithmic_bytes(cfg, seqs)
    kv_bytes = sum(seqs) * cfg.nkv * 2 * cfg.D
    out = torch.empty((cfg.B * cfg.s1, cfg.nq, cfg.D), dtype=torch.bfloat16, device="cuda")

    def run(splits, steps, warmup, rot):
        need, nsplit = binding.workspace_size(cfg.B, cfg.s1, cfg.nq, cfg.nkv, cfg.D, cfg.block_size,
                                              cfg.max_blocks_per_seq, cfg.s2_tile, splits)
        ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
        wall, region, ev = time_calls(binding, rot, steps, warmup, splits, out, ws)
        return wall, region, ev, nsplit

    if args.pmc_mode:
        # fixed, short: decode calls then one plain device copy of known size
        run(args.splits, 20, 5, sets)
        src = torch.empty(256 * 1024 * 1024, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_mode": True, "decode_calls": 25, "copy_bytes": src.numel(), "copies": 5,
                          "algorithmic_bytes_per_call": nbytes}))
        return

    if args.sweep_splits:
        for sp in [int(x) for x in args.sweep_splits.split(",")]:
            wall, _, ev, nsplit = run(sp, args.steps, args.warmup, sets)
            med = ev[len(ev) // 2]
            print(json.dumps({"splits": nsplit, "median_us": round(med * 1e3, 2),
                              "gb_s": round(nbytes / (med * 1e-3) / 1e9, 1),
                              "wall_us_per_call": round(wall / args.steps * 1e6, 2)}), flush=True)
        return

    host0 = {k: (v.cpu() if hasattr(v, "cpu") else v) for k, v in sets[0].items()}
    wall, region, ev, nsplit = run(args.splits, args.steps, args.warmup, sets)
    ms_per_step = wall / args.steps * 1e3
    mean_ev = sum(ev) / len(ev)
    med_ev = ev[len(ev) // 2]
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (region * 1e-3) / 1e9
    _, region_warm, _, _ = run(args.splits, max(20, args.steps // 4), 5, sets[:1])
    warm = nbytes / (region_warm * 1e-3) / 1e9
    traffic, traffic_note = pmc_traffic()

    line = {
        "metric": "achieved HBM GB/s (% of 8 TB/s peak) + decode calls/s, FP8 paged GQA decode",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (products exact, fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "s1": cfg.s1, "nq": cfg.nq, "nkv": cfg.nkv, "D": cfg.D,
                   "block_size": cfg.block_size, "s2_tile": cfg.s2_tile, "seq_lens": "U[1024,8192] seed 1",
                   "total_tokens": sum(seqs), "path": "whole-row" if args.splits == 0 else f"per-head, {nsplit} splits",
                   "causal": bool(args.causal),
                   "rotating_input_sets": len(sets),
                   "algorithmic_bytes_per_call": nbytes},
        "calls_per_s": round(1.0 / (ms_per_step * 1e-3), 1),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "kv_gb_s": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "query_head_tokens_per_s": round(cfg.B * cfg.s1 * cfg.nq / (ms_per_step * 1e-3), 1),
        "event_us_per_call_timed_region": round(region * 1e3, 2),
        "event_us_per_call": {"mean": round(mean_ev * 1e3, 2), "median": round(med_ev * 1e3, 2),
                              "p10": round(ev[len(ev) // 10] * 1e3, 2), "p90": round(ev[(9 * len(ev)) // 10] * 1e3, 2),
                              "note": "separate pass, one event pair around each call"},
        "warm_cache_gb_s": round(warm, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic), "traffic_note": traffic_note,
                     "kernel": ("pa::decode_rows_kernel + pa::merge_rows_kernel" if args.splits == 0
                                else "pa::decode_kernel" + (" + pa::combine_kernel" if nsplit > 1 else ""))},
    }
    # over-fetch by whole cache blocks: a sequence's last block is read in full (masked past its length)
    blk_tokens = sum((sq + cfg.block_size - 1) // cfg.block_size * cfg.block_size for sq in seqs)
    block_bytes = nbytes + (blk_tokens - sum(seqs)) * cfg.nkv * (2 * cfg.D + 4)
    line["block_granular"] = {"bytes_per_call": block_bytes, "ratio_to_algorithmic": round(block_bytes / nbytes, 4),
                              "gb_s": round(block_bytes / (region * 1e-3) / 1e9, 2)}
    # secondary: the two contractions (S = Q K^T and P V) as bf16 MFMA work on exact FP8 codes
    flops = 4 * cfg.D * cfg.s1 * cfg.nq * sum(seqs)
    line["mfma_secondary"] = {
        "flop_per_call": flops, "achieved": round(flops / (region * 1e-3) / 1e12, 2), "peak": 2500.0,
        "unit": "TFLOP/s", "frac": round(flops / (region * 1e-3) / 1e12 / 2500.0, 4),
        "note": "analytic, exact lengths; the work executed with query rows padded to 16 is counted by "
                "SQ_INSTS_VALU_MFMA_MOPS_BF16 in profiles/mfma_counters_glm45_b32_and_mla.md"}
    if not args.no_secondary and args.config == 1 and not args.causal and args.splits == 0:
        del sets
        torch.cuda.empty_cache()
        line["secondary"] = secondary_entries(args)
        sets = None
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, host0, seqs, args.cpu_target_s)
    print(json.dumps(line), flush=True)


def prefill_config():
    """A chunked-prefill workload of the GLM-4.5 head layout: 128 new tokens at the
    end of each of 4 sequences of U[2048, 8192] tokens, causal (position s sees the
    first seq - 128 + 1 + s tokens)."""
    from fp8_paged_kv_amd import synth
    return synth.GqaConfig("prefill-chunk-b4-s1-128-nq96-nkv8-seq2k-8k", B=4, s1=128, nq=96, nkv=8,
                           seq_range=(2048, 8192), s2_tile=512, num_blocks=4 * 64, max_blocks_per_seq=64,
                           outlier_frac=0.01, seed=5)


def causal_flops(cfg, seqs):
    """Both contractions over the tokens each query row sees (causal limits)."""
    G = cfg.nq // cfg.nkv
    tok = 0
    for sq in seqs:
        for s in range(cfg.s1):
            tok += max(0, min(sq - cfg.s1 + 1 + s, sq))
    return 4 * cfg.D * G * cfg.nkv * tok


def prefill_path(cfg):
    """Whether the library runs this shape on its prefill kernel (the header's rule for
    num_splits = 0): at least 128 query rows per KV head, s2_tile 128 / 256 / 512 and at
    least 64 (batch, KV head, 128-row tile) workgroups."""
    rows = cfg.s1 * cfg.nq // cfg.nkv
    return rows >= 128 and cfg.s2_tile in (128, 256, 512) and cfg.B * cfg.nkv * ((rows + 127) // 128) >= 64


def whole_row_path(cfg):
    """Whether the library runs this shape on its whole-row path (the header's rule for
    num_splits = 0): at most 32 query rows per KV head, or more in blocks of 32 with
    s2_tile up to 512; at most 1024 (batch, KV-head group, row block) units."""
    rows = cfg.s1 * cfg.nq // cfg.nkv
    rbk = 1 if rows <= 32 else (rows + 31) // 32
    hg = 2 if cfg.nkv % 2 == 0 else 1
    tile_ok = cfg.s2_tile in (128, 256, 512) or (cfg.s2_tile == 1024 and rows <= 16)
    return tile_ok and cfg.B * rbk * (cfg.nkv // hg) <= 1024


def measure_gqa(cfg_id, causal, steps, warmup, rotate, cfg=None):
    """Event-timed decode calls on one GQA workload (rotating input sets):
    algorithmic bytes, us per call and the HBM roofline fraction (the bf16 MFMA one
    for prefill-length s1, where the contractions dominate)."""
    import torch
    from fp8_paged_kv_amd import binding, synth
    cfg = cfg or synth.CONFIGS[cfg_id]
    sets, seqs = make_sets(cfg, rotate)
    for st in sets:
        st["causal"] = causal
    nbytes = synth.gqa_algorithmic_bytes(cfg, seqs)
    out = torch.empty((cfg.B * cfg.s1, cfg.nq, cfg.D), dtype=torch.bfloat16, device="cuda")
    need, _ = binding.workspace_size(cfg.B, cfg.s1, cfg.nq, cfg.nkv, cfg.D, cfg.block_size, cfg.max_blocks_per_seq,
                                     cfg.s2_tile, 0)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    _, region, ev = time_calls(binding, sets, steps, warmup, 0, out, ws)
    del sets
    torch.cuda.empty_cache()
    gbs = nbytes / (region * 1e-3) / 1e9
    rows = cfg.s1 * cfg.nq // cfg.nkv
    entry = {"workload": cfg.name + ("-causal" if causal else ""), "algorithmic_bytes_per_call": nbytes,
             "us_per_call": round(region * 1e3, 2), "median_us": round(ev[len(ev) // 2] * 1e3, 2),
             "calls_per_s": round(1e3 / region, 1),
             "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gbs / HBM_PEAK_GBS, 4)},
             "kernel": ("pa::prefill_kernel" if prefill_path(cfg)
                        else "pa::decode_rows_kernel + pa::merge_rows_kernel" if whole_row_path(cfg)
                        else "pa::decode_kernel")}
    if rows > 32:
        flops = causal_flops(cfg, seqs) if causal else 4 * cfg.D * cfg.s1 * cfg.nq * sum(seqs)
        tf = flops / (region * 1e-3) / 1e12
        entry["flop_per_call"] = flops
        entry["roofline"] = {"bound": "mfma", "achieved": round(tf, 1), "peak": 2500.0, "unit": "TFLOP/s",
                             "frac": round(tf / 2500.0, 4), "hbm_gb_s": round(gbs, 1),
                             "note": "exact FP8 products on the bf16 MFMA: its dense peak"}
    return entry


def measure_mla(kv_split, steps, warmup, rotate):
    """Event-timed MLA sparse decode calls: bf16 MFMA roofline (and HBM beside it)."""
    import torch
    from fp8_paged_kv_amd import binding, synth
    cfg = synth.CONFIGS[4]
    first = synth.make_mla_inputs(cfg, device="cuda")
    seqs = first["kv_act_seqs"].cpu().tolist()
    sets = [first] + [synth.make_mla_inputs(cfg, device="cuda", seed=1000 + 17 * i + cfg.seed, seq_lens=seqs)
                      for i in range(1, max(1, rotate))]
    if kv_split:
        sets = [synth.mla_kv_split(st) for st in sets]
    run_one = binding.mla_decode_kv_split_inputs if kv_split else binding.mla_decode_inputs
    out = torch.empty((cfg.B * cfg.s1 * cfg.nq, 512), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(binding.mla_workspace_size(cfg.B, cfg.s1, cfg.nq, cfg.topk, cfg.s2_tile), dtype=torch.uint8,
                     device="cuda")

    def call(i, stream):
        run_one(sets[i % len(sets)], out=out, workspace=ws, stream=stream)

    wall, region, ev = _timed(call, steps, warmup)
    nbytes = synth.mla_algorithmic_bytes(cfg, seqs)
    ntok = sum(cfg.s1 * cfg.nkv * min(int(q), cfg.topk) for q in seqs)
    flops = 2 * (576 + 512) * (cfg.nq // cfg.nkv) * ntok          # S = [qn|qr].K and P.V, per query head
    tf = flops / (region * 1e-3) / 1e12
    return dict(cfg=cfg, seqs=seqs, wall=wall, region=region, ev=ev, nbytes=nbytes, ntok=ntok, flops=flops,
                entry={"workload": cfg.name + ("-kv-split" if kv_split else ""),
                       "algorithmic_bytes_per_call": nbytes, "flop_per_call": flops,
                       "us_per_call": round(region * 1e3, 2), "median_us": round(ev[len(ev) // 2] * 1e3, 2),
                       "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": 2500.0, "unit": "TFLOP/s",
                                    "frac": round(tf / 2500.0, 4),
                                    "hbm_gb_s": round(nbytes / (region * 1e-3) / 1e9, 1)},
                       "kernel": "pa::mla_decode_kernel + pa::mla_merge_kernel"})


def secondary_entries(args):
    """The other workloads, each timed like the headline (event-timed region over
    rotating input sets), for the same JSON line."""
    st, wu, rot = args.secondary_steps, 10, max(1, args.rotate)
    sec = {}
    for key, cid, causal in (("config2", 2, False), ("config3", 3, False), ("config3_causal", 3, True)):
        sec[key] = measure_gqa(cid, causal, st, wu, rot)
    sec["prefill_causal_s1_128"] = measure_gqa(None, True, max(5, st // 10), 3, 1, cfg=prefill_config())
    sec["config4_mla"] = measure_mla(False, st, wu, rot)["entry"]
    sec["config4_mla_kv_split"] = measure_mla(True, st, wu, rot)["entry"]
    return sec


def run_ceiling(args):
    """Read-only probes beside the decode on config 1's workload: the bytes the decode
    must read, in its paged layout, with nothing computed (the access pattern's
    ceiling), and a contiguous read of a buffer of the same size."""
    import ctypes
    import torch
    from fp8_paged_kv_amd import binding, build, synth
    lib_path = build.PROBE_LIB
    if not os.path.exists(lib_path):
        sys.exit(f"{lib_path} is missing: build it with fp8_paged_kv_amd.build.build_probe()")
    P = ctypes.CDLL(lib_path)
    vp = ctypes.c_void_p
    P.pa_probe_paged_read.argtypes = [vp] * 5 + [ctypes.c_int] * 6 + [vp, vp]
    P.pa_probe_paged_read.restype = ctypes.c_int
    P.pa_probe_contiguous_read.argtypes = [vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, vp, vp]
    P.pa_probe_contiguous_read.restype = ctypes.c_int
    cfg = synth.CONFIGS[1]
    sets, seqs = make_sets(cfg, max(1, args.rotate))
    nbytes = synth.gqa_algorithmic_bytes(cfg, seqs)
    blk_tok = sum((q + 127) // 128 * 128 for q in seqs)
    paged_bytes = blk_tok * cfg.nkv * (2 * cfg.D + 4)             # whole blocks of K, V and k_scale
    sink = torch.empty(cfg.B * cfg.nkv // 2 * cfg.max_blocks_per_seq, dtype=torch.int32, device="cuda")

    def paged_probe(pgrid, nh=2):
        def call(i, stream):
            d = sets[i % len(sets)]
            rc = P.pa_probe_paged_read(d["k_cache"].data_ptr(), d["k_scale"].data_ptr(), d["v_cache"].data_ptr(),
                                       d["block_table"].data_ptr(), d["kv_act_seqs"].data_ptr(), cfg.B, cfg.nkv,
                                       cfg.max_blocks_per_seq, cfg.num_blocks, pgrid, nh, sink.data_ptr(),
                                       ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"probe launch failed: {rc}")
        return _timed(call, args.steps, args.warmup)[1]

    paged = {f"one workgroup per block of {nh} KV heads": paged_probe(0, nh) for nh in (2, 4, 8)}
    for pg in (256, 1024):
        paged[f"{pg} persistent workgroups, 2 KV heads per item"] = paged_probe(pg)
    n16 = paged_bytes // 16
    bufs = [torch.empty(n16 * 16, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(max(1, args.rotate))]
    csink = torch.empty(256 * 16, dtype=torch.int32, device="cuda")

    def contiguous_probe(grid, unroll):
        def call(i, stream):
            rc = P.pa_probe_contiguous_read(bufs[i % len(bufs)].data_ptr(), n16, grid, unroll, csink.data_ptr(),
                                            ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"probe launch failed: {rc}")
        return _timed(call, args.steps, args.warmup)[1]

    contig = {}
    for grid in (256, 512, 1024, 2048, 4096):
        for unroll in (4, 8):
            contig[f"{grid} workgroups, {unroll} loads in flight"] = contiguous_probe(grid, unroll)
    out = torch.empty((cfg.B, cfg.nq, cfg.D), dtype=torch.bfloat16, device="cuda")
    need, _ = binding.workspace_size(cfg.B, 1, cfg.nq, cfg.nkv, cfg.D, 128, cfg.max_blocks_per_seq, cfg.s2_tile, 0)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    _, r_dec, _ = time_calls(binding, sets, args.steps, args.warmup, 0, out, ws)
    line = {
        "metric": "read-only ceilings of the paged decode's access pattern, GB/s",
        "config": {"workload": cfg.name, "rotating_input_sets": len(sets), "algorithmic_bytes_per_call": nbytes,
                   "paged_probe_bytes": paged_bytes},
        "paged_probe": {k: {"us": round(v * 1e3, 2), "gb_s": round(paged_bytes / (v * 1e-3) / 1e9, 1)}
                        for k, v in paged.items()},
        "paged_probe_note": "items = (batch, group of KV heads, valid 128-token block): the group's K and V "
                            "slices of the 128 token rows and its k_scale words, XOR-folded, nothing computed",
        "best_paged_2_heads_gb_s": round(paged_bytes / (paged["one workgroup per block of 2 KV heads"] * 1e-3) / 1e9,
                                         1),
        "contiguous_probe": {k: {"us": round(v * 1e3, 2), "gb_s": round(paged_bytes / (v * 1e-3) / 1e9, 1)}
                             for k, v in contig.items()},
        "contiguous_probe_note": "the same byte count read from one contiguous buffer, 16-byte loads",
        "best_paged_gb_s": round(paged_bytes / (min(paged.values()) * 1e-3) / 1e9, 1),
        "best_contiguous_gb_s": round(paged_bytes / (min(contig.values()) * 1e-3) / 1e9, 1),
        "decode": {"us": round(r_dec * 1e3, 2), "gb_s": round(nbytes / (r_dec * 1e-3) / 1e9, 1),
                   "kernel": "pa::decode_rows_kernel + pa::merge_rows_kernel"},
    }
    print(json.dumps(line), flush=True)


def run_valu_rates(args):
    """Issue rate of the VALU instructions that turn FP8 codes into MFMA operands, from
    the probe library: every SIMD of the chip busy with 8 waves (2048 workgroups of
    256 threads), each wave running 8 independent chains; event-timed."""
    import ctypes
    import torch
    from fp8_paged_kv_amd import build
    P = ctypes.CDLL(build.PROBE_LIB)
    P.pa_probe_valu_rate.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    P.pa_probe_valu_rate.restype = ctypes.c_int
    names = ["v_mul_f32", "v_cvt_pk_f32_fp8 (2 codes -> 2 FP32)", "v_cvt_pk_bf16_f32 (2 FP32 -> 2 BF16, RNE)",
             "v_cvt_scalef32_pk_bf16_fp8 (2 codes -> 2 BF16)", "v_perm_b32", "v_fma_f32"]
    grid, threads, iters = 2048, 256, 4096
    simds = torch.cuda.get_device_properties(0).multi_processor_count * 4
    sink = torch.empty(grid * threads, dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for op, name in enumerate(names):
        for _ in range(2):
            if P.pa_probe_valu_rate(op, grid, threads, iters, sink.data_ptr(), st) != 0:
                sys.exit(f"probe launch failed for {name}")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            P.pa_probe_valu_rate(op, grid, threads, iters, sink.data_ptr(), st)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps * 1e-3
        per_simd = grid * (threads // 64) * iters * 8 / simds       # wave instructions per SIMD
        res[name] = {"ns_per_wave_instruction_per_simd": round(t / per_simd * 1e9, 4),
                     "cycles_at_2.4GHz": round(t / per_simd * 2.4e9, 2)}
    base = res[names[0]]["ns_per_wave_instruction_per_simd"]
    for name in names:
        res[name]["relative_to_v_mul_f32"] = round(res[name]["ns_per_wave_instruction_per_simd"] / base, 2)
    print(json.dumps({"metric": "VALU issue rate, wave64 instructions", "simds": simds,
                      "waves_per_simd": grid * (threads // 64) / simds, "rates": res}), flush=True)


def run_lds_patterns(args):
    """LDS read rate of lane address patterns, from the probe library: 2 workgroups of
    8 waves per CU, each wave issuing iters x 8 independent reads; event-timed.  Bytes
    per cycle per CU at 2.4 GHz; a pattern whose lanes collide in banks reads slower."""
    import ctypes
    import torch
    from fp8_paged_kv_amd import build
    P = ctypes.CDLL(build.PROBE_LIB)
    P.pa_probe_lds_pattern.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_void_p]
    P.pa_probe_lds_pattern.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid, iters = 2 * cus, 2048
    sink = torch.empty(grid * 512, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cases = [(0, 0, 16), (0, 0, 8)]
    cases += [(1, s, 16) for s in (256, 264, 272, 288, 320, 384, 512)]
    cases += [(2, s, 16) for s in (128, 136, 256, 272)]
    cases += [(3, s, 16) for s in (16, 32, 64, 128, 136, 144, 272)]
    cases += [(3, s, 8) for s in (8, 16, 128, 136)]
    names = {0: "16 lane", 1: "(lane % 16) stride + 16 (lane / 16)", 2: "(lane / 4) stride + 16 (lane % 4)",
             3: "lane stride"}
    rows = []
    for pat, stride, width in cases:
        for _ in range(2):
            if P.pa_probe_lds_pattern(pat, stride, width, grid, iters, sink.data_ptr(), st) != 0:
                sys.exit(f"probe launch failed for pattern {pat} stride {stride}")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            P.pa_probe_lds_pattern(pat, stride, width, grid, iters, sink.data_ptr(), st)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps * 1e-3
        nbytes = grid * 8 * iters * 8 * 64 * width
        rows.append({"pattern": names[pat].replace("16", str(width)) if pat == 0 else names[pat], "stride": stride,
                     "bytes_per_lane": width, "bytes_per_clk_per_cu": round(nbytes / t / cus / 2.4e9, 1)})
    print(json.dumps({"metric": "LDS read rate by lane address pattern", "cus": cus, "rows": rows}), flush=True)


def run_fp8_mfma(args):
    """What gfx950's FP8 MFMA (v_mfma_f32_16x16x32_fp8_fp8) returns for 16x16x32
    products of E4M3 codes, against the exact FP64 sums, beside the bf16 MFMA on
    the same codes decoded exactly (the contraction the decode kernels use)."""
    import ctypes
    import numpy as np
    import torch
    from fp8_paged_kv_amd import build, synth
    P = ctypes.CDLL(build.PROBE_LIB)
    vp = ctypes.c_void_p
    P.pa_probe_fp8_mfma.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp]
    P.pa_probe_fp8_mfma.restype = ctypes.c_int
    g = torch.Generator().manual_seed(11)

    def finite_codes(shape):
        c = torch.randint(0, 254, shape, generator=g, dtype=torch.int32)
        return (c + (c >= 0x7F).to(torch.int32)).to(torch.uint8)

    def e4m3(x):
        return x.to(torch.float8_e4m3fn).view(torch.uint8)

    cases = {}
    n = 256
    cases["uniform codes (all finite E4M3 values)"] = (finite_codes((n, 16, 32)), finite_codes((n, 16, 32)))
    a = torch.randn((n, 16, 32), generator=g)
    b = torch.randn((n, 16, 32), generator=g)
    cases["N(0,1) rows scaled to amax 448"] = (e4m3(a / a.abs().amax(-1, keepdim=True) * 448),
                                              e4m3(b / b.abs().amax(-1, keepdim=True) * 448))
    # one large product per group of 8 beside seven small ones of the same sign
    a = torch.full((n, 16, 32), 2.0 ** -3)
    b = torch.full((n, 16, 32), 2.0 ** -3)
    a[:, :, ::8] = 448.0
    b[:, :, ::8] = 448.0
    cases["one 448x448 product and seven 2^-6 products per group of 8"] = (e4m3(a), e4m3(b))
    # the GLM-4.5-shaped workload's own operands: query codes q / q_scale and key codes from the cache,
    # 32-channel slices, 12 query heads of a KV head (+4 repeated) against 16 tokens
    cfg = synth.CONFIGS[1]
    inp = synth.make_gqa_inputs(cfg)
    q8 = e4m3(inp["q"].float() / inp["q_scale"][..., None])          # [B, nq, 128]
    k8 = inp["k_cache"]                                                # [nb, 128, nkv, 128]
    G = cfg.nq // cfg.nkv
    table = inp["block_table"]
    aa, bb = [], []
    for i in range(n):
        bi, h, sl = i % cfg.B, (i // cfg.B) % cfg.nkv, (i // (cfg.B * cfg.nkv)) % 4
        heads = [h * G + (j % G) for j in range(16)]
        blk = int(table[bi, 0])
        aa.append(q8[bi, heads, 32 * sl:32 * sl + 32])
        bb.append(k8[blk, 16 * (i % 8):16 * (i % 8) + 16, h, 32 * sl:32 * sl + 32])
    cases["GLM-4.5-shaped workload: query codes x key codes (outlier channels x20)"] = (torch.stack(aa),
                                                                                        torch.stack(bb))
    report = {}
    for name, (ca, cb) in cases.items():
        ca, cb = ca.contiguous(), cb.contiguous()
        cnt = ca.shape[0]
        da, db = ca.cuda(), cb.cuda()
        c = torch.empty((cnt, 16, 16), device="cuda")
        cr = torch.empty_like(c)
        rc = P.pa_probe_fp8_mfma(da.data_ptr(), db.data_ptr(), c.data_ptr(), cr.data_ptr(), cnt,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"probe launch failed: {rc}")
        torch.cuda.synchronize()
        va = ca.view(torch.float8_e4m3fn).double().numpy()
        vb = cb.view(torch.float8_e4m3fn).double().numpy()
        exact = np.einsum("nik,njk->nij", va, vb)
        mag = np.einsum("nik,njk->nij", np.abs(va), np.abs(vb))        # sum of |products|
        got, ref = c.cpu().double().numpy(), cr.cpu().double().numpy()
        scale = np.maximum(np.abs(exact), 1e-30)
        e8, eb = np.abs(got - exact), np.abs(ref - exact)
        i8 = np.unravel_index(int(np.argmax(e8 / scale)), e8.shape)
        report[name] = {
            "products": int(exact.size),
            "fp8_mfma": {"max_rel_err": float((e8 / scale).max()), "max_err_over_sum_abs": float((e8 / mag).max()),
                         "frac_rel_err_above_1e-3": float(((e8 / scale) > 1e-3).mean()),
                         "frac_inexact": float((e8 > 0).mean()),
                         "worst": {"exact": float(exact[i8]), "fp8_mfma": float(got[i8])}},
            "bf16_mfma_on_decoded_codes": {"max_rel_err": float((eb / scale).max()),
                                           "max_err_over_sum_abs": float((eb / mag).max()),
                                           "frac_inexact": float((eb > 0).mean())},
        }
    print(json.dumps({"metric": "FP8 MFMA vs exact sums, 16x16x32 products of E4M3 codes", "cases": report}),
          flush=True)


def _pct(a, q):
    import numpy as np
    return round(float(np.percentile(a, q)), 2)


def run_phases(args):
    """Per-workgroup phase times of the decode (--config 1-3, whole-row kernel) or the
    MLA decode (--config 4), read from the phase-stamp build of the library
    (libpa_fp8_phases.so: the same kernels and results, plus s_memrealtime stamps)."""
    import ctypes
    import numpy as np
    import torch
    from fp8_paged_kv_amd import binding, build, synth
    if not os.path.exists(build.PHASES_LIB):
        sys.exit(f"{build.PHASES_LIB} is missing: build it with fp8_paged_kv_amd.build.build_phases()")
    binding._lib = None
    binding.LIB_PATH = build.PHASES_LIB
    L = binding.lib()
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    us = 0.01                                                  # s_memrealtime ticks (100 MHz) -> us
    calls = max(4, min(args.steps, 20))
    if args.config == 4:
        L.pa_fp8_phases_mla.restype = ctypes.c_void_p
        ptr = L.pa_fp8_phases_mla()
        cfg = synth.CONFIGS[4]
        first = synth.make_mla_inputs(cfg, device="cuda")
        seqs = first["kv_act_seqs"].cpu().tolist()
        sets = [first] + [synth.make_mla_inputs(cfg, device="cuda", seed=1000 + 17 * i + cfg.seed, seq_lens=seqs)
                          for i in range(1, max(1, args.rotate))]
        out = torch.empty((cfg.B * cfg.nq, 512), dtype=torch.bfloat16, device="cuda")
        ws = torch.zeros(binding.mla_workspace_size(cfg.B, 1, cfg.nq, cfg.topk, cfg.s2_tile), dtype=torch.uint8,
                         device="cuda")
        grid = cfg.B * cfg.s1 * ((cfg.topk + cfg.s2_tile - 1) // cfg.s2_tile) * (cfg.nq // 32)
        names = ["rows and queries staged", "score pass", "wait for the tile maxima", "softmax, P to LDS",
                 "P.V pass", "partial writes"]
        for i in range(args.warmup):
            binding.mla_decode_inputs(sets[i % len(sets)], out=out, workspace=ws)
        torch.cuda.synchronize()
        buf = np.zeros(4096 * 8, dtype=np.uint64)
        rows = []
        for i in range(calls):
            binding.mla_decode_inputs(sets[i % len(sets)], out=out, workspace=ws)
            torch.cuda.synchronize()
            hip.hipMemcpy(buf.ctypes.data, ptr, buf.nbytes, 2)
            rows.append(buf.reshape(4096, 8)[:grid, :7].astype(np.int64).copy())
        st = np.stack(rows)                                    # [calls, wg, 7]
        t0 = st[:, :, 0].min(axis=1, keepdims=True)
        d = np.diff(st, axis=2) * us
        phases = {n: {"mean": round(float(d[:, :, k].mean()), 2), "p10": _pct(d[:, :, k], 10),
                      "p90": _pct(d[:, :, k], 90)} for k, n in enumerate(names)}
        start, end = (st[:, :, 0] - t0) * us, (st[:, :, 6] - t0) * us
        line = {"metric": "per-workgroup phase times, us", "config": {"workload": cfg.name, "calls": calls,
                                                                        "workgroups": grid},
                "kernel": "pa::mla_decode_kernel", "phases": phases,
                "dispatch_ramp": {"mean": round(float(start.mean()), 2), "max": round(float(start.max()), 2)},
                "workgroup_end": {"mean": round(float(end.mean()), 2), "p90": _pct(end, 90),
                                  "max": round(float(end.max(axis=1).mean()), 2)}}
        print(json.dumps(line), flush=True)
        return
    L.pa_fp8_phases_rows.restype = ctypes.c_void_p
    ptr = L.pa_fp8_phases_rows()
    cfg = synth.CONFIGS[args.config]
    sets, seqs = make_sets(cfg, max(1, args.rotate))
    out = torch.empty((cfg.B * cfg.s1, cfg.nq, cfg.D), dtype=torch.bfloat16, device="cuda")
    need, _ = binding.workspace_size(cfg.B, cfg.s1, cfg.nq, cfg.nkv, cfg.D, cfg.block_size, cfg.max_blocks_per_seq,
                                     cfg.s2_tile, 0)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    for i in range(args.warmup):
        binding.decode_inputs(sets[i % len(sets)], out=out, workspace=ws)
    torch.cuda.synchronize()
    buf = np.zeros(256 * 16, dtype=np.uint64)
    rows = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    call_us = []
    for i in range(calls):
        e0.record()
        binding.decode_inputs(sets[i % len(sets)], out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        call_us.append(e0.elapsed_time(e1) * 1e3)
        hip.hipMemcpy(buf.ctypes.data, ptr, buf.nbytes, 2)
        rows.append(buf.reshape(256, 16).astype(np.int64).copy())
    st = np.stack(rows)                                        # [calls, 256, 16]
    live = st[:, :, 5] > 0                                     # workgroups that had work
    t0 = st[:, :, 0].min(axis=1, keepdims=True)
    ramp = (st[:, :, 0] - t0) * us
    pro = (st[:, :, 1] - st[:, :, 0]) * us
    first = (st[:, :, 7] - st[:, :, 1]) * us
    loop = (st[:, :, 2] - st[:, :, 1]) * us
    qc, ends = st[:, :, 3] * us, st[:, :, 4] * us
    stream = loop - qc - ends
    steps, segs = st[:, :, 5], st[:, :, 6]
    end = (st[:, :, 2] - t0) * us
    span = end.max(axis=1)

    def stat(a):
        a = a[live]
        return {"mean": round(float(a.mean()), 2), "p10": _pct(a, 10), "p90": _pct(a, 90)}

    per_step = (stream[live] / np.maximum(steps[live], 1))
    line = {"metric": "per-workgroup phase times of the decode, us",
            "config": {"workload": cfg.name, "calls": calls, "workgroups_with_work": int(live[0].sum())},
            "kernel": "pa::decode_rows_kernel",
            "call_us_event": round(float(np.mean(call_us)), 2),
            "decode_kernel_span_us": round(float(span.mean()), 2),
            "dispatch_ramp": stat(ramp), "prologue": stat(pro),
            "prologue_parts": {"lengths_staged": stat((st[:, :, 8] - st[:, :, 0]) * us),
                               "cost_prefix": stat((st[:, :, 9] - st[:, :, 8]) * us),
                               "first_unit_found": stat((st[:, :, 10] - st[:, :, 9]) * us),
                               "table_entries_arrived": stat((st[:, :, 11] - st[:, :, 10]) * us),
                               "first_loads_issued": stat((st[:, :, 1] - st[:, :, 11]) * us)},
            "first_step_data_after_prologue": stat(first),
            "query_conversion_total": stat(qc), "segment_ends_total": stat(ends), "streaming": stat(stream),
            "steps": {"mean": round(float(steps[live].mean()), 1), "min": int(steps[live].min()),
                      "max": int(steps[live].max())},
            "segments": {"mean": round(float(segs[live].mean()), 2), "max": int(segs[live].max())},
            "us_per_streaming_step": {"mean": round(float(per_step.mean()), 3), "p10": _pct(per_step, 10),
                                      "p90": _pct(per_step, 90)},
            "workgroup_end": stat(end),
            "tail_after_mean_end": round(float((span - np.array([e[l].mean() for e, l in zip(end, live)])).mean()), 2)}
    print(json.dumps(line), flush=True)


def run_mla(args):
    """The MLA-style sparse decode workload (B=16, nq=128, topk 2048, seq 4k-32k)."""
    m = measure_mla(args.kv_split, args.steps, args.warmup, args.rotate)
    cfg, ms = m["cfg"], m["wall"] / args.steps * 1e3
    line = {
        "metric": "MLA sparse decode, algorithmic GB/s and bf16 TFLOP/s",
        "value": round(m["nbytes"] / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 MFMA on dequantised fp8 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": m["entry"]["workload"], "B": cfg.B, "s1": cfg.s1, "nq": cfg.nq, "nkv": cfg.nkv,
                   "topk": cfg.topk, "s2_tile": cfg.s2_tile, "algorithmic_bytes_per_call": m["nbytes"],
                   "flop_per_call": m["flops"],
                   "layout": "kv_split (three tensors)" if args.kv_split else "packed 672-byte rows"},
        "event_us_per_call_timed_region": round(m["region"] * 1e3, 2),
        "event_us_per_call": {"mean": round(sum(m["ev"]) / len(m["ev"]) * 1e3, 2),
                              "median": round(m["ev"][len(m["ev"]) // 2] * 1e3, 2),
                              "note": "separate pass, one event pair around each call"},
        "tflop_s": m["entry"]["roofline"]["achieved"],
        "roofline": dict(m["entry"]["roofline"], traffic=None, kernel=m["entry"]["kernel"]),
        # a gathered row is 656 used bytes of a 672-byte cache row
        "row_stride": {"bytes_per_call": m["nbytes"] + m["ntok"] * (672 - 656),
                       "ratio_to_algorithmic": round((m["nbytes"] + m["ntok"] * (672 - 656)) / m["nbytes"], 4)},
    }
    print(json.dumps(line), flush=True)


def _time(fn, steps, warmup):
    return _timed(lambda i, stream: fn(stream), steps, warmup)


def run_scatter(args):
    """The FP8 KV-cache writer: every token of the GLM-4.5-shaped workload
    (B=32, lengths U[1024, 8192], 8 KV heads, D=128) written into its
    2048-block pool in the decode's layout, int32 slots; plus one decode step
    (one new token per sequence)."""
    import torch
    from fp8_paged_kv_amd import binding, synth
    cfg = synth.CONFIGS[1]
    pre = synth.prefill_slots(cfg, device="cuda")
    slots = pre["slots"]
    T, H, D = int(slots.numel()), cfg.nkv, cfg.D
    g = torch.Generator(device="cuda").manual_seed(7)
    key = torch.randint(0, 256, (T, H, D), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    value = torch.randint(0, 256, (T, H, D), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    ks = torch.rand((T, H), generator=g, device="cuda")
    shape = (cfg.num_blocks, cfg.block_size, H, D)
    kc = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    vc = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    ksc = torch.zeros(shape[:3], device="cuda")

    def call(stream):
        binding.scatter_kv_cache(key, value, kc, vc, slots, ks, ksc, "BSND", stream=stream)

    wall, region, ev = _time(call, args.steps, args.warmup)
    per_tok = 2 * (2 * H * D + 4 * H) + 4          # read + write of both rows and the scales, the slot
    nbytes = T * per_tok
    # decode step: one token per sequence, at position seq_b (the next slot of each table row)
    seqs = pre["seqs"].tolist()
    step_slots = torch.tensor([int(pre["block_table"][b, (s - 1) // 128]) * 128 + (s - 1) % 128
                               for b, s in enumerate(seqs)], dtype=torch.int32, device="cuda")
    kd, vd, sd = key[: cfg.B].contiguous(), value[: cfg.B].contiguous(), ks[: cfg.B].contiguous()

    def step(stream):
        binding.scatter_kv_cache(kd, vd, kc, vc, step_slots, sd, ksc, "BSND", stream=stream)

    _, _, ev_step = _time(step, args.steps, args.warmup)
    ms = wall / args.steps * 1e3
    mean = region
    achieved = nbytes / (mean * 1e-3) / 1e9
    line = {
        "metric": "FP8 KV-cache writer, algorithmic GB/s", "value": round(nbytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8 (fp8 codes copied)",
        "data": "synthetic",
        "config": {"workload": "kv-writer-prefill-glm45-b32-nkv8-seq1k-8k", "num_tokens": T, "num_head": H,
                   "head_size": D, "num_blocks": cfg.num_blocks, "block_size": cfg.block_size, "layout": "BSND",
                   "slot_bits": 32, "algorithmic_bytes_per_call": nbytes},
        "event_us_per_call_timed_region": round(region * 1e3, 2),
        "event_us_per_call": {"mean": round(sum(ev) / len(ev) * 1e3, 2), "median": round(ev[len(ev) // 2] * 1e3, 2),
                              "note": "separate pass, one event pair around each call"},
        "decode_step_us": {"tokens": cfg.B, "median": round(ev_step[len(ev_step) // 2] * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "pa::scatter_kv_kernel<int, 0>"},
    }
    print(json.dumps(line), flush=True)


def run_epilog(args):
    """KvCompressEpilog, quant mode 1 (e8m0 scales, roundScale): 131072 bf16 rows
    of the MLA latent width d = 576 (512 nope + 64 rope) written into a
    1024 x 128-row cache of 649-byte rows (the 648 bytes a row needs, one spare)."""
    import torch
    from fp8_paged_kv_amd import binding, synth
    cfg = synth.EpilogConfig("epilog-bench", num_tokens=131072, d=576, block_num=1024, block_size=128,
                             head_dim=649, quant_mode=1, round_scale=True, seed=9)
    inp = synth.make_epilog_inputs(cfg, device="cuda")

    def call(stream):
        binding.epilog_inputs(inp, stream=stream)

    wall, region, ev = _time(call, args.steps, args.warmup)
    row_bytes = (cfg.d - 64) + 128 + (cfg.d - 64) // 64
    nbytes = cfg.num_tokens * (2 * cfg.d + row_bytes + 4)          # read x and the slot, write the row
    ms = wall / args.steps * 1e3
    mean = region
    achieved = nbytes / (mean * 1e-3) / 1e9
    line = {
        "metric": "KvCompressEpilog mode 1, algorithmic GB/s", "value": round(nbytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 -> fp8 e4m3 codes, fp32 scale arithmetic", "data": "synthetic",
        "config": {"workload": "kv-compress-epilog-mode1-d576-tokens131072", "num_tokens": cfg.num_tokens,
                   "d": cfg.d, "block_num": cfg.block_num, "block_size": cfg.block_size, "head_dim": cfg.head_dim,
                   "quant_mode": 1, "round_scale": True, "algorithmic_bytes_per_call": nbytes},
        "event_us_per_call_timed_region": round(region * 1e3, 2),
        "event_us_per_call": {"mean": round(sum(ev) / len(ev) * 1e3, 2), "median": round(ev[len(ev) // 2] * 1e3, 2),
                              "note": "separate pass, one event pair around each call"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "pa::kv_compress_epilog_kernel<int, 1>"},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
