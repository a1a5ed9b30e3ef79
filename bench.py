#!/usr/bin/env python3
"""Benchmark of FastGen's hot path on one MI355X.

Default workload: the Llama-1-65B-shaped stack -- 80 attention layers x 64 heads,
head_dim 128, bf16, batch 16, prompt 2048, T = 0.95, r_l = r_f = 0.3, 1024
decode steps.  One step is the whole path over that batch:
  prompt phase: for every layer, fg_profile (row statistics sweep, column-sum
      sweep, top-k + recovery + policy) and fg_compact (plan, gather refilling
      that layer's cache);
  decode: 1024 generated tokens, each decoded through every layer's cache in
      turn (fg_decode_step: split-K partials, then combine / append / evict).
Inputs (per layer Q, K, V; 16 decode inputs per layer, cycled; the full class
sequence of the generated tokens) are drawn on the device and resident in HBM
before timing.  The prompt phase is captured as one HIP graph and the decode
loop as graphs of 16 tokens each (``--mode eager`` launches every call from
Python); before timing, one replayed step is checked bit for bit against an
eager run.

Prints ONE JSON line.  ``value`` is profile+compact prompt tokens/s over the
whole stack (B * n / prompt-phase time, the median over the timed steps; by
default 5 steps after 2 warm-ups); decode tokens/s (B * steps / decode time,
likewise), per-kernel figures, the roofline of the dominant kernel, whole-phase
fractions of the MFMA and HBM ceilings, the chip's measured ceilings and the
CPU oracle (sampled heads, extrapolated) are reported beside it.
``--config 1`` (or ``--layer L`` of a stack) times one attention layer instead,
with the optional full-cache, prompt-attention and decode-stability blocks.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synth import inputs as syn  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_MFMA_PEAK_TFLOPS = 157.3
# v_exp_f32 at half rate: 8 lanes / clock / SIMD x 4 SIMD x 256 CU x 2.4 GHz (1e12 exponentials / s)
EXP_PEAK_T_PER_S = 8 * 4 * 256 * 2.4e9 / 1e12
METRIC = "profile+compact prompt tok/s & decode tok/s on 1 MI355X; % MFMA / HBM peak"


# ---------------------------------------------------------------- CPU baseline (the oracle)
def _oracle_head(args):
    """Profile + compact (and optionally decode) one KV head with the oracle, 1 BLAS thread."""
    from threadpoolctl import threadpool_limits
    from oracle import fastgen_ref as ref
    spec_id, layer, h, do_decode = args
    spec = syn.CONFIGS[spec_id]
    with threadpool_limits(1):
        li = syn.make_layer(spec, layer, heads=[h])
        G = spec.group
        t0 = time.perf_counter()
        pr = ref.profile_head(li.Q[0, :G], li.K[0, 0], li.token_class[0], spec.r_l, spec.r_f, spec.T[0])
        ref.compact_head(li.K[0, 0], li.V[0, 0], pr.kept)
        t1 = time.perf_counter()
        td = 0.0
        if do_decode:
            ds = syn.make_decode_stream(spec, layer, heads=[h])
            t2 = time.perf_counter()
            ref.decode_incremental(li.K[0, 0], li.V[0, 0], li.token_class[0], pr.F, pr.w_l, pr.policy,
                                   ds.q[:, 0, :G], ds.k[:, 0, 0], ds.v[:, 0, 0], ds.new_class[:, 0])
            td = time.perf_counter() - t2
    return t1 - t0, td


def cpu_baseline(spec: syn.ConfigSpec, sample_heads: int, layer: int = 0) -> dict:
    """Time the oracle on a sample of KV heads over a fork pool (run before the GPU is touched)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    cores = min(16, len(os.sched_getaffinity(0)))
    heads = list(range(min(sample_heads, spec.n_kv_heads)))
    ctx = mp.get_context("fork")
    def progress(it, what):
        out = []
        for k, r in enumerate(it):
            out.append(r)
            print(f"[cpu] {what}: {k + 1} of {len(heads)} KV heads", file=sys.stderr, flush=True)
        return out

    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx) as ex:
        t0 = time.perf_counter()
        res = progress(ex.map(_oracle_head, [(spec.cfg_id, layer, h, False) for h in heads]), "profile+compact")
        w_prompt = time.perf_counter() - t0
        t0 = time.perf_counter()
        res_d = progress(ex.map(_oracle_head, [(spec.cfg_id, layer, h, True) for h in heads]), "with decode")
        w_both = time.perf_counter() - t0
    scale = spec.batch * spec.n_kv_heads / len(heads)
    prompt_tok_s = spec.batch * spec.seq_len / (w_prompt * scale)
    w_dec = max(w_both - w_prompt, 1e-9)
    decode_tok_s = spec.batch * spec.decode_steps / (w_dec * scale)
    return {"value": prompt_tok_s, "unit": "prompt tok/s (profile+compact)", "cores": cores, "kind": "oracle",
            "decode_tok_s": decode_tok_s,
            "sample": f"{len(heads)} of {spec.n_kv_heads} KV heads of the layer (profile+compact, then also "
                      f"{spec.decode_steps} decode steps), fp64 numpy oracle with 1 BLAS thread per worker over "
                      f"{cores} forked workers; wall times scaled by {scale:g} to the whole layer",
            "cpu_seconds": float(sum(a + b for a, b in res_d) + sum(a for a, _ in res))}


# ---------------------------------------------------------------- HBM traffic from counters
CALIB_BYTES = 256 << 20
CALIB_BLOCKS = 1000          # the calibration copy's grid (1000 x 256 threads), unlike any other copy launched
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


KERNEL_SOURCES = {
    "profile_rowstats": "profile_kernels.hip", "profile_colsums": "profile_kernels.hip",
    "profile_select": "select_kernels.hip", "compact_gather": "compact_kernels.hip",
    "decode_partials": "decode_kernels.hip", "decode_merge": "decode_kernels.hip",
}


def kernel_sources_digest(kernel=None) -> str:
    """Digest of the HIP sources a kernel is built from (its own file and the shared headers; every
    source when ``kernel`` is None): counter-derived traffic is reported only for the same sources."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "adaptive_kv_cache_fg_amd", "csrc")
    own = KERNEL_SOURCES.get(kernel)
    for name in sorted(os.listdir(csrc)):
        if name.endswith(".h") or (name.endswith(".hip") and (own is None or name == own)):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of ``kernel`` in ``workload`` from profiles/traffic.json (FETCH_SIZE +
    WRITE_SIZE, scaled by the calibration copy), or None when absent, taken on another workload,
    or taken on other sources of that kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get("workloads", {}).get(workload)
    if not entry or kernel not in entry.get("bytes_per_launch", {}):
        return None
    if entry.get("sources_digest", {}).get(kernel) != kernel_sources_digest(kernel):
        return None
    return float(entry["bytes_per_launch"][kernel])


def calibration_copy(torch, fg) -> None:
    """A copy of known size (CALIB_BYTES read, CALIB_BYTES written) with a grid of its own, outside
    any timed region: under rocprofv3 --pmc, what FETCH_SIZE / WRITE_SIZE read for it scales the
    counters of the other kernels (record_traffic)."""
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    fg.peak_copy(src, dst, False, CALIB_BLOCKS)
    torch.cuda.synchronize()
    del src, dst


# ---------------------------------------------------------------- GPU path
def upload(torch, x, dtype):
    if dtype == "bf16":
        bits = syn.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def prompt_attention(torch, fg, Qd, Kd, Vd, cls, spec, T, sweep_flops, reps=20) -> dict:
    """Profiling's marginal cost over the prompt attention it rides on (graph-replayed calls)."""
    B, Hq, n, d = Qd.shape
    O = torch.empty_like(Qd)

    def time_graph(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        e[0].record()
        for _ in range(reps):
            g.replay()
        e[1].record()
        torch.cuda.synchronize()
        del g
        return 1e3 * e[0].elapsed_time(e[1]) / reps

    attn_us = time_graph(lambda: fg.attention(Qd, Kd, Vd, out=O))
    fused_us = time_graph(lambda: fg.profile(Qd, Kd, cls, spec.r_l, spec.r_f, T, V=Vd))
    prof_us = time_graph(lambda: fg.profile(Qd, Kd, cls, spec.r_l, spec.r_f, T))
    # the optional per-row level bins (a third sweep; not part of the profiling step)
    lprof = fg.profile(Qd, Kd, cls, spec.r_l, spec.r_f, T, want_lse=True)
    bins_us = time_graph(lambda: fg.row_bins(Qd, Kd, cls, lprof))
    # the fused call gives the same attention output and the same decisions as the two separate calls
    fused = fg.profile(Qd, Kd, cls, spec.r_l, spec.r_f, T, V=Vd)
    plain = fg.profile(Qd, Kd, cls, spec.r_l, spec.r_f, T)
    fg.attention(Qd, Kd, Vd, out=O)
    torch.cuda.synchronize()
    if not (torch.equal(fused.out, O) and torch.equal(fused.policy, plain.policy)):
        raise RuntimeError("fused profiling disagrees with attention + profiling")
    # per-kernel times of one eager fused call
    fg.timing_read()
    fg.timing_enable(True)
    fg.profile(Qd, Kd, cls, spec.r_l, spec.r_f, T, V=Vd)
    torch.cuda.synchronize()
    fg.timing_enable(False)
    kern = {k: 1e3 * ms for k, ms in fg.timing_read()}
    attn_flops = 2 * sweep_flops                          # S = Q K^T and O = P V over the causal pairs
    sdpa_us = None
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        G = Hq // Kd.shape[1]
        Ke = Kd.repeat_interleave(G, dim=1) if G > 1 else Kd
        Ve = Vd.repeat_interleave(G, dim=1) if G > 1 else Vd
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            sdpa = lambda: torch.nn.functional.scaled_dot_product_attention(Qd, Ke, Ve, is_causal=True)  # noqa: E731
            sdpa()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            e[0].record()
            for _ in range(reps):
                sdpa()
            e[1].record()
            torch.cuda.synchronize()
            sdpa_us = 1e3 * e[0].elapsed_time(e[1]) / reps
        del Ke, Ve
    except Exception:                                    # no fused torch attention for this shape
        sdpa_us = None
    ach = attn_flops / (kern["attention"] * 1e-6) / 1e12
    return {
        "attention_us": attn_us, "profile_attention_us": fused_us, "profile_alone_us": prof_us,
        "profiling_marginal_us": fused_us - attn_us,
        "profiling_marginal_frac": (fused_us - attn_us) / attn_us,
        "fusion_saving_us": attn_us + prof_us - fused_us,
        "attention_kernel": {"avg_us": kern["attention"], "algorithmic_flops": attn_flops, "achieved": ach,
                             "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / BF16_MFMA_PEAK_TFLOPS},
        "fused_kernels_us": kern,
        "row_bins_us": bins_us,
        "row_bins_score_tflops": sweep_flops / (bins_us * 1e-6) / 1e12,
        "torch_sdpa_us": sdpa_us,
        "prompt_tok_s_attention_only": B * n / (attn_us * 1e-6),
        "prompt_tok_s_attention_with_profiling": B * n / (fused_us * 1e-6),
        "note": "graph-replayed calls; marginal = fg_profile_attention - fg_attention; torch_sdpa_us is "
                "torch's fused causal attention on the same tensors (K, V repeated per query head), "
                "launched eagerly",
    }


def decode_stability(torch, fg, Kd, Vd, cls, prof, qs, ks, vs, ncs, spec, T) -> dict:
    """Accumulated attention at the prompt step against the generated tokens' attention, over full
    caches (every head keeps every key), tracked on the device step by step with fg_decode_track."""
    B, Hkv, n, d = Kd.shape
    Hq = qs.shape[2]
    steps = qs.shape[0]
    e = Kd.element_size()
    full = fg.apply_head_map(prof, torch.full((Hkv,), 4, dtype=torch.uint8, device="cuda"))
    cache = fg.compact(Kd, Vd, cls, full, Hq, max_new_tokens=steps, max_new_kept=steps)
    score = cache.track_init(prof)
    cls_all = torch.cat([cls, ncs.t()], dim=1).contiguous()             # classes of positions 0 .. n+steps-1
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    bins = torch.empty((steps, B, Hkv, 5), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    fg.timing_read()
    fg.timing_enable(True)
    for t in range(steps):
        cache.decode_step(qs[t], ks[t], vs[t], ncs[t], out=out)
        cache.track(qs[t], cls_all, prof.freq_mask, score, level_bins=bins[t])
    torch.cuda.synchronize()
    fg.timing_enable(False)
    track_ms = [ms for k, ms in fg.timing_read() if k == "decode_track"]
    b = bins.cpu().numpy().astype(np.float64)                           # [steps, B, Hkv, 5]
    R = prof.recovery.cpu().numpy().astype(np.float64)
    share_prompt = np.diff(np.concatenate([np.zeros((B, Hkv, 1)), R], axis=-1), axis=-1)
    tv_mean_share = 0.5 * np.abs(b.mean(axis=0) - share_prompt).sum(axis=-1)   # [B, Hkv]
    tv_step = 0.5 * np.abs(b - share_prompt[None]).sum(axis=-1)                  # [steps, B, Hkv]
    pol = prof.policy.cpu().numpy().astype(np.int64)
    retained = np.take_along_axis(np.cumsum(b, axis=-1), pol[None, :, :, None], axis=-1)[..., 0]
    # frequent set re-ranked by the scores accumulated through generation (full caches: row j holds
    # position j of its head), against the prompt's
    k_f = int(np.floor(spec.r_f * n))
    sc = score.cpu().numpy()
    ro = cache.t["row_offset"].cpu().numpy()
    F0 = prof.frequent()
    overlap = []
    for hd in range(B * Hkv):
        s_h = sc[ro[hd]: ro[hd] + n + steps]
        top = np.lexsort((np.arange(len(s_h)), -s_h))[:k_f]              # largest first, ties to the lower index
        overlap.append(len(set(top.tolist()) & set(np.flatnonzero(F0[hd // Hkv, hd % Hkv]).tolist())) / max(k_f, 1))
    rows = float(B * Hkv * n + B * Hkv * (steps + 1) / 2.0)
    track_bytes = rows * (2 * d * e + 12)
    avg_us = 1e3 * float(np.mean(track_ms))

    # the frequent set re-ranked during generation (local + frequent heads) against the static
    # policy: the same stream through two adaptive caches, one decoded with fg_decode_step_dynamic
    # (scores tracked after every step), one with fg_decode_step
    dyn = fg.compact(Kd, Vd, cls, prof, Hq, max_new_tokens=steps, max_new_kept=steps)
    sta = fg.compact(Kd, Vd, cls, prof, Hq, max_new_tokens=steps, max_new_kept=steps)
    dscore = dyn.track_init(prof)
    out2 = torch.empty_like(out)
    torch.cuda.synchronize()
    fg.timing_read()
    fg.timing_enable(True)
    for t in range(steps):
        dyn.decode_step_dynamic(qs[t], ks[t], vs[t], ncs[t], cls_all, dscore, out=out)
        dyn.track(qs[t], cls_all, prof.freq_mask, dscore)
        sta.decode_step(qs[t], ks[t], vs[t], ncs[t], out=out2)
    torch.cuda.synchronize()
    fg.timing_enable(False)
    recs = fg.timing_read()
    merges = [ms for k, ms in recs if k == "decode_merge"]       # dynamic and static alternate
    kd, ks_ = dyn.kept_positions(), sta.kept_positions()
    moved = int(sum(len(set(a.tolist()) - set(b.tolist())) for a, b in zip(kd, ks_)))
    n_pol3 = int(np.sum(pol == 3))
    dynamic = {
        "local_frequent_heads": n_pol3,
        "keys_kept_that_the_static_policy_dropped": moved,
        "merge_us_dynamic": 1e3 * float(np.mean(merges[0::2])) if merges else None,
        "merge_us_static": 1e3 * float(np.mean(merges[1::2])) if merges else None,
        "note": "adaptive caches; per-launch events; the dynamic merge launch also scans the permanent rows of "
                "each local + frequent head for the weakest frequent key",
    }
    return {
        "steps": steps,
        "tv_distance_mean_share": {"mean": float(tv_mean_share.mean()), "max": float(tv_mean_share.max())},
        "tv_distance_per_step": {"mean": float(tv_step.mean()), "p95": float(np.percentile(tv_step, 95))},
        "prompt_policy_retained_ge_T": float(np.mean(retained >= T - 1e-6)),
        "prompt_policy_retained_min": float(retained.min()),
        "frequent_set_overlap_after_generation": {"mean": float(np.mean(overlap)), "min": float(np.min(overlap))},
        "dynamic_frequent_set": dynamic,
        "track_kernel": {"avg_us": avg_us, "algorithmic_bytes": track_bytes,
                         "achieved": track_bytes / (avg_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": track_bytes / (avg_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         "note": "three launches per step (events around the whole call); K of every cached row "
                                 "read twice, position and score read, score written"},
        "note": "full caches (every head keeps every key); level shares of each generated token's attention vs "
                "the prompt's per-level recovery increments; total-variation distance; retained = attention "
                "the prompt-chosen policy's levels get at each decode step",
    }


def bench_layer(args, spec: syn.ConfigSpec, cpu) -> dict:
    """One attention layer of a workload (its profile, compaction and decode loop), with the
    optional measurement blocks (full-cache baseline, prompt attention, decode stability)."""
    import torch
    from adaptive_kv_cache_fg_amd import fastgen as fg

    li = syn.make_layer(spec, args.layer)
    ds = syn.make_decode_stream(spec, args.layer)
    steps_dec = spec.decode_steps
    Qd, Kd, Vd = upload(torch, li.Q, spec.dtype), upload(torch, li.K, spec.dtype), upload(torch, li.V, spec.dtype)
    cls = torch.from_numpy(li.token_class).cuda()
    qs = upload(torch, ds.q, spec.dtype)
    ks = upload(torch, ds.k, spec.dtype)
    vs = upload(torch, ds.v, spec.dtype)
    ncs = torch.from_numpy(ds.new_class).cuda()
    outs = torch.empty((steps_dec, spec.batch, spec.n_q_heads, spec.head_dim), dtype=torch.float32, device="cuda")
    max_new_kept = int(max(np.count_nonzero(ds.new_class[:, b]) for b in range(spec.batch)))
    T = float(args.T) if args.T is not None else spec.T[0]
    B, Hq, n, d = li.Q.shape

    def prompt_phase(reuse=None, check=True):
        # refilling a cache: the profile writes its policies straight into the cache's buffer
        prof = fg.profile(Qd, Kd, cls, spec.r_l, spec.r_f, T,
                          policy_out=None if reuse is None else reuse.t["policy"])
        cache = fg.compact(Kd, Vd, cls, prof, Hq, max_new_tokens=steps_dec, max_new_kept=max_new_kept,
                           reuse=reuse, check=check)
        return prof, cache

    def decode_eager(cache):
        for t in range(steps_dec):
            cache.decode_step(qs[t], ks[t], vs[t], ncs[t], out=outs[t])

    # one eager pass allocates the cache and the decode workspace
    prof, cache = prompt_phase()
    decode_eager(cache)
    graph = pgraph_prompt = None
    prof_g = None
    if args.mode == "graph":
        # the prompt phase (profile, then the compaction refilling the cache's buffers without a
        # host read of the totals) and the whole 256-token decode loop, each as one HIP graph
        torch.cuda.synchronize()
        pgraph_prompt = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pgraph_prompt):
            prof_g, _ = prompt_phase(reuse=cache, check=False)
        prompt_phase(reuse=cache)                            # eager: resets the host-side position
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode_eager(cache)
        torch.cuda.synchronize()

    def one_step(ev=None):
        if ev is not None:
            ev[0].record()
        if pgraph_prompt is not None:
            pgraph_prompt.replay()
            res = (prof_g, cache)
        else:
            res = prompt_phase(reuse=cache)
        if ev is not None:
            ev[1].record()
        if graph is not None:
            graph.replay()
        else:
            decode_eager(cache)
        if ev is not None:
            ev[2].record()
        return res

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    # correctness guard on the timed configuration: the replayed prompt phase and decode loop
    # equal an eager rerun
    ref_out = outs.clone()
    ref_prof = [x.clone() for x in (prof_g.policy, prof_g.cum, prof_g.recovery)] if prof_g is not None else None
    eprof, _ = prompt_phase(reuse=cache)
    decode_eager(cache)
    torch.cuda.synchronize()
    if not torch.equal(ref_out, outs):
        raise RuntimeError("graph replay and eager decode disagree")
    if ref_prof is not None and not all(torch.equal(a, b) for a, b in
                                        zip(ref_prof, (eprof.policy, eprof.cum, eprof.recovery))):
        raise RuntimeError("graph replay and eager prompt phase disagree")
    if cache.error_bits() != 0:
        raise RuntimeError("cache error bits set")
    fg.timing_read()                                         # drop anything pending
    fg.timing_enable(True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    last = None
    for s in range(args.steps):
        last = one_step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fg.timing_enable(False)
    recs = fg.timing_read()
    if pgraph_prompt is not None:
        # the prompt kernels on one eager pass with the library's events around each launch
        torch.cuda.synchronize()
        fg.timing_enable(True)
        prompt_phase(reuse=cache)
        torch.cuda.synchronize()
        fg.timing_enable(False)
        recs += fg.timing_read()
    partials_us = None
    if graph is not None:
        # launches inside the graph carry no per-launch events.  The split-K launch alone
        # (fg_decode_partials: read-only on the cache) for the same 256 steps from the same cache
        # state, as a graph timed by events around its replay; the merge launch on one eager pass
        # with the library's events around each launch.
        prompt_phase(reuse=cache)
        torch.cuda.synchronize()
        pgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pgraph):
            for t in range(steps_dec):
                cache.decode_partials(qs[t])
        pgraph.replay()
        pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        pe[0].record()
        pgraph.replay()
        pe[1].record()
        torch.cuda.synchronize()
        partials_us = 1e3 * pe[0].elapsed_time(pe[1]) / steps_dec
        del pgraph
        fg.timing_read()
        fg.timing_enable(True)
        decode_eager(cache)
        torch.cuda.synchronize()
        fg.timing_enable(False)
        recs += fg.timing_read()

    prompt_ms = float(np.median([evs[s][0].elapsed_time(evs[s][1]) for s in range(args.steps)]))
    decode_ms = float(np.median([evs[s][1].elapsed_time(evs[s][2]) for s in range(args.steps)]))
    ms_per_step = wall * 1e3 / args.steps
    prompt_tok_s = B * n / (prompt_ms * 1e-3)
    decode_tok_s = B * steps_dec / (decode_ms * 1e-3)

    # per-kernel averages: the library's HIP events around each launch (prompt kernels over the
    # timed steps; decode kernels over the eager pass above when the timed decode is a graph)
    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    kstats = {}
    for k, v in per.items():
        reps = 1 if (graph is not None and k.startswith("decode")) or (pgraph_prompt is not None and
                                                                       not k.startswith("decode")) else args.steps
        kstats[k] = {"launches_per_step": len(v) / reps, "avg_us": 1e3 * float(np.mean(v)),
                     "total_us_per_step": 1e3 * float(np.sum(v)) / reps, "timing": "events around each launch"}
    if partials_us is not None:
        kstats["decode_partials"].update(
            avg_us=partials_us, total_us_per_step=partials_us * steps_dec,
            timing=f"events around a graph of {steps_dec} fg_decode_partials launches (per-launch events "
                   f"in an eager pass: {kstats['decode_partials']['avg_us']:.2f} us)")
        merge_us = 1e3 * decode_ms / steps_dec - partials_us
        kstats["decode_merge"].update(
            avg_us=merge_us, total_us_per_step=merge_us * steps_dec,
            timing=f"graph decode step minus the graph-timed partials launch (per-launch events in an "
                   f"eager pass: {kstats['decode_merge']['avg_us']:.2f} us)")

    # algorithmic work per launch
    prof, cache = last
    e = 2 if spec.dtype == "bf16" else 4
    pairs = n * (n + 1) // 2
    sweep_flops = B * Hq * 2 * d * pairs
    kept = cache.kept_count.cpu().numpy().astype(np.int64)
    pol = prof.policy.cpu().numpy().reshape(-1)
    gather_bytes = int(np.sum(kept * (2 * d * e) * 2 + 4 * kept) + B * spec.n_kv_heads * (n + n / 8))
    # decode: cache rows in use grow by the appended tokens; mean over the steps
    len_start = kept.copy()
    cls_new = ds.new_class
    grow = np.zeros_like(len_start, dtype=np.float64)
    for hd in range(len(pol)):
        b = hd // spec.n_kv_heads
        p = int(pol[hd])
        nc = cls_new[:, b]
        if p == 4:
            add = np.arange(steps_dec)
        elif p == 3:
            add = np.cumsum(nc != 0) - (nc != 0)                 # punct appended; ring size fixed
        elif p >= 1:
            add = np.cumsum(nc != 0) - (nc != 0)
        else:
            add = np.cumsum(nc == 1) - (nc == 1)
        grow[hd] = float(np.mean(add))
    mean_rows = float(np.sum(len_start + grow))
    Hkv = spec.n_kv_heads
    G = Hq // Hkv
    # partials launch: cache rows (K, V, position tag) and q; merge launch: the new k, v rows and
    # q (the new token's own score), the partial states, the fp32 output
    dec_bytes = mean_rows * (2 * d * e + 4) + B * Hq * d * e
    merge_bytes = B * Hkv * 2 * d * e + B * Hq * d * (e + 4) + cache.c.n_work * G * (d + 2) * 4
    step_bytes = mean_rows * (2 * d * e + 4) + B * Hkv * 2 * d * e + B * Hq * d * (e + 4)
    kstats["decode_step"] = {"launches_per_step": float(steps_dec), "avg_us": 1e3 * decode_ms / steps_dec,
                             "total_us_per_step": 1e3 * decode_ms,
                             "note": "whole decode step (both launches and the gaps between them)"}
    kinfo = {
        "profile_rowstats": ("mfma", sweep_flops, "TFLOP/s"),
        "profile_colsums": ("mfma", sweep_flops, "TFLOP/s"),
        "compact_gather": ("hbm", gather_bytes, "GB/s"),
        "decode_partials": ("hbm", dec_bytes, "GB/s"),
        "decode_merge": ("hbm", merge_bytes, "GB/s"),
        "decode_step": ("hbm", step_bytes, "GB/s"),
    }
    peak_mfma = BF16_MFMA_PEAK_TFLOPS if spec.dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS
    for k, (bound, units, unit) in kinfo.items():
        if k not in kstats:
            continue
        avg_s = kstats[k]["avg_us"] * 1e-6
        if bound == "mfma":
            ach = units / avg_s / 1e12
            kstats[k].update(bound="mfma", achieved=ach, peak=peak_mfma, unit=unit, frac=ach / peak_mfma,
                             algorithmic_flops=units)
        else:
            ach = units / avg_s / 1e9
            kstats[k].update(bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit=unit, frac=ach / HBM_PEAK_GBS,
                             algorithmic_bytes=units)
    dominant = max((k for k in kinfo if k in kstats and k != "decode_step"),
                   key=lambda k: kstats[k]["total_us_per_step"])
    dk = kstats[dominant]
    roofline = {"bound": dk["bound"], "achieved": dk["achieved"], "peak": dk["peak"], "unit": dk["unit"],
                "frac": dk["frac"], "traffic": measured_traffic(dominant, layer_workload_key(spec, args.layer, T)),
                "kernel": dominant}

    # full-cache baseline (outside the timed region): the same decode loop over caches that keep
    # every key (the full policy forced for every head), against the adaptive caches above
    full = None
    if not args.no_full_baseline:
        fprof = fg.apply_head_map(fg.profile(Qd, Kd, cls, spec.r_l, spec.r_f, T),
                                  torch.full((spec.n_kv_heads,), 4, dtype=torch.uint8, device="cuda"))
        fcache = fg.compact(Kd, Vd, cls, fprof, Hq, max_new_tokens=steps_dec, max_new_kept=max_new_kept)
        fouts = torch.empty_like(outs)

        def full_decode():
            for t in range(steps_dec):
                fcache.decode_step(qs[t], ks[t], vs[t], ncs[t], out=fouts[t])

        full_decode()
        fg.compact(Kd, Vd, cls, fprof, Hq, max_new_tokens=steps_dec, max_new_kept=max_new_kept, reuse=fcache)
        torch.cuda.synchronize()
        fgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(fgraph):
            full_decode()
        fts = []
        for _ in range(max(3, min(args.steps, 10))):
            fg.compact(Kd, Vd, cls, fprof, Hq, max_new_tokens=steps_dec, max_new_kept=max_new_kept,
                       reuse=fcache, check=False)
            fe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            fe[0].record()
            fgraph.replay()
            fe[1].record()
            torch.cuda.synchronize()
            fts.append(fe[0].elapsed_time(fe[1]))
        del fgraph
        full_ms = float(np.median(fts))
        full_rows = float(B * spec.n_kv_heads * n + B * spec.n_kv_heads * (steps_dec - 1) / 2.0)
        kept_rows = mean_rows
        full = {
            "decode_tok_s": B * steps_dec / (full_ms * 1e-3),
            "decode_speedup": (full_ms / steps_dec) / (decode_ms / steps_dec),
            "kv_bytes_full": full_rows * 2 * d * e,
            "kv_bytes_adaptive": kept_rows * 2 * d * e,
            "kv_pruned_fraction": 1.0 - kept_rows / full_rows,
            "note": "same decode loop over caches keeping every key (the full policy forced for every head), "
                    "graph-replayed; KV bytes are "
                    "mean rows in use over the steps x 2*d*e",
        }

    # the prompt's attention output with the profiling riding on it (outside the timed region):
    # attention alone, attention fused with the profiling, the profiling alone, each captured as
    # a HIP graph and timed over replays; torch's own causal attention on the same tensors as
    # context.  Profiling's marginal cost is fused minus attention alone.
    attn = None
    if spec.dtype == "bf16" and not args.no_attention:
        attn = prompt_attention(torch, fg, Qd, Kd, Vd, cls, spec, T, sweep_flops)
        # one layer's generation: fused prompt pass, compaction, every decode step
        gen_us = attn["profile_attention_us"] + max(0.0, 1e3 * prompt_ms - attn["profile_alone_us"]) + 1e3 * decode_ms
        attn["generation_us"] = gen_us
        attn["profiling_share_of_generation"] = attn["profiling_marginal_us"] / gen_us

    # stability of accumulated attention from the prompt into generation (outside the timed region)
    stab = None
    if not args.no_stability:
        stab = decode_stability(torch, fg, Kd, Vd, cls, prof, qs, ks, vs, ncs, spec, T)

    calibration_copy(torch, fg)

    result = {
        "metric": METRIC,
        "value": prompt_tok_s,
        "unit": "prompt tok/s (profile+compact)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype,
        "data": "synthetic (seeded Llama-shaped post-RoPE Q/K/V with planted head types)",
        "config": {"workload": f"{spec.name}: 1 attention layer"
                               f"{f' (layer {args.layer} of {spec.layers})' if spec.layers > 1 else ''}, "
                               f"B={B}, Hq={Hq}, Hkv={spec.n_kv_heads}, n={n}, d={d}, {spec.dtype}, T={T}, "
                               f"r_l={spec.r_l}, r_f={spec.r_f}, {steps_dec} decode steps",
                   "batch": B, "seq_len": n, "decode_steps": steps_dec, "layer": args.layer},
        "decode_tok_s": decode_tok_s, "mode": args.mode,
        "prompt_ms": prompt_ms, "decode_ms": decode_ms,
        "policy_histogram": np.bincount(pol, minlength=5).tolist(),
        "kept_fraction": float(kept.sum() / (B * spec.n_kv_heads * n)),
        "roofline": roofline,
        "full_cache_baseline": full,
        "prompt_attention": attn,
        "decode_stability": stab,
        "kernels": kstats,
        "cpu_baseline": cpu,
    }
    return result


# ---------------------------------------------------------------- workload keys
def layer_workload_key(spec: syn.ConfigSpec, layer: int, T: float) -> str:
    return f"{spec.name}/layer{layer}/T{T}"


def stack_workload_key(spec: syn.ConfigSpec, T: float, layers: int, steps: int) -> str:
    return f"{spec.name}/stack{layers}/T{T}/steps{steps}"


# ---------------------------------------------------------------- CPU baseline of a stack (the oracle)
def _oracle_stack_head(args):
    """Oracle profile + compact of one (layer, batch entry, KV head), then its decode over the
    workload's generated tokens; per-head wall seconds of each part (1 BLAS thread)."""
    from threadpoolctl import threadpool_limits
    from oracle import fastgen_ref as ref
    spec_id, layer, b, h, steps = args
    spec = syn.CONFIGS[spec_id]
    G = spec.group
    with threadpool_limits(1):
        li = syn.make_layer(spec, layer, batch=[b], heads=[h])
        ds = syn.make_decode_stream(spec, layer, steps, batch=[b], heads=[h])
        t0 = time.perf_counter()
        pr = ref.profile_head(li.Q[0, :G], li.K[0, 0], li.token_class[0], spec.r_l, spec.r_f, spec.T[0])
        ref.compact_head(li.K[0, 0], li.V[0, 0], pr.kept)
        t1 = time.perf_counter()
        ref.decode_incremental(li.K[0, 0], li.V[0, 0], li.token_class[0], pr.F, pr.w_l, pr.policy,
                               ds.q[:, 0, :G], ds.k[:, 0, 0], ds.v[:, 0, 0], ds.new_class[:, 0])
        t2 = time.perf_counter()
    return layer, t1 - t0, t2 - t1, pr.policy


def cpu_baseline_stack(spec: syn.ConfigSpec, layers_layers: int) -> dict:
    """The oracle on every KV head of batch entry 0 in two sample layers, one outer (layer 0:
    broad / local heads) and one middle (layer L/2: special-dominated), timed per head in a fork
    pool (run before the GPU is touched).  The whole stack is extrapolated from the per-head CPU
    seconds: each outer and middle layer of the stack costs what its sample layer costs per batch
    entry, times the batch; wall time = CPU seconds / cores (the heads are independent)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    cores = min(16, len(os.sched_getaffinity(0)))
    L = layers_layers
    outer, middle = 0, L // 2
    steps = spec.decode_steps
    jobs = [(spec.cfg_id, layer, 0, h, steps) for layer in (outer, middle) for h in range(spec.n_kv_heads)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx) as ex:
        res = []
        for k, r in enumerate(ex.map(_oracle_stack_head, jobs)):
            res.append(r)
            if k % 16 == 15:
                print(f"[cpu] {k + 1} of {len(jobs)} sampled heads", file=sys.stderr, flush=True)
    wall = time.perf_counter() - t0
    prof_s = {outer: 0.0, middle: 0.0}
    dec_s = {outer: 0.0, middle: 0.0}
    for layer, tp, td, _ in res:
        prof_s[layer] += tp
        dec_s[layer] += td
    n_outer = sum(1 for l in range(L) if l < 4 or l >= L - 4)
    n_middle = L - n_outer
    cpu_prompt = spec.batch * (n_outer * prof_s[outer] + n_middle * prof_s[middle])
    cpu_decode = spec.batch * (n_outer * dec_s[outer] + n_middle * dec_s[middle])
    return {"value": spec.batch * spec.seq_len / (cpu_prompt / cores), "unit": "prompt tok/s (profile+compact)",
            "cores": cores, "kind": "oracle", "extrapolated": True,
            "decode_tok_s": spec.batch * steps / (cpu_decode / cores),
            "sample": f"fp64 numpy oracle (1 BLAS thread per worker, {cores} forked workers) on all "
                      f"{spec.n_kv_heads} KV heads of batch entry 0 in layer {outer} (outer) and layer {middle} "
                      f"(middle), profile+compact then {steps} decode steps each, inputs from the host "
                      f"generator of the same recipe; extrapolated linearly in heads to {L} layers "
                      f"({n_outer} outer, {n_middle} middle) x {spec.batch} batch entries, wall = CPU s / cores",
            "sample_cpu_seconds": float(sum(r[1] + r[2] for r in res)), "sample_wall_seconds": wall,
            "whole_stack_cpu_hours": (cpu_prompt + cpu_decode) / 3600.0}


# ---------------------------------------------------------------- the chip's own ceilings
def chip_peaks(torch, fg) -> dict:
    """Micro-benchmarks (libfastgen's fg_peak_*): bf16 MFMA issue rate, the MFMA rate beside the
    sweeps' softmax work in other waves of the same SIMDs, v_exp_f32 rate, a 1 GiB HBM copy and a
    4 GiB read-only stream, each the best over a few occupancies, events around repeated launches."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        for _ in range(reps):
            fn()
        e[1].record()
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) * 1e-3 / reps

    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    ops = torch.randn(8192, generator=g, device="cuda").to(torch.bfloat16)
    mfma = []
    for per_cu in (1, 2, 4):
        blocks = per_cu * cus
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        iters = 8000
        flops = blocks * 4 * 4 * 32768 * iters
        t = timed(lambda: fg.peak_mfma_bf16(ops, out, iters, blocks))
        mfma.append({"waves_per_simd": per_cu, "tflops": flops / t / 1e12, "ms": t * 1e3})
    mix = []
    for per_cu in (1, 2, 3):                       # 512-thread workgroups: 2, 4, 6 waves per SIMD, half MFMA
        blocks = per_cu * cus
        out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
        iters = 8000
        flops = blocks * 4 * 4 * 32768 * iters
        t = timed(lambda: fg.peak_mfma_softmax(ops, out, iters, blocks))
        mix.append({"waves_per_simd": 2 * per_cu, "tflops": flops / t / 1e12, "ms": t * 1e3})
    exps = []
    for per_cu in (2, 4, 8):
        blocks = per_cu * cus
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        iters = 40000
        n = blocks * 256 * 8 * iters
        t = timed(lambda: fg.peak_exp(out, iters, blocks))
        exps.append({"waves_per_simd": per_cu, "t_exp_per_s": n / t / 1e12, "ms": t * 1e3})
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    copies = []
    for nt in (False, True):
        for per_cu in (4, 8):
            blocks = per_cu * cus
            t = timed(lambda: fg.peak_copy(src, dst, nt, blocks), reps=10)
            copies.append({"nontemporal": nt, "blocks_per_cu": per_cu, "gbs": 2 * nbytes / t / 1e9})
    del src, dst
    rbytes = 4 << 30
    rsrc = torch.empty(rbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    reads = []
    for nt in (False, True):
        for per_cu in (16, 32, 64):
            blocks = per_cu * cus
            words = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
            t = timed(lambda: fg.peak_read(rsrc, words, nt, blocks), reps=10)
            reads.append({"nontemporal": nt, "blocks_per_cu": per_cu, "gbs": rbytes / t / 1e9})
    del rsrc
    best = lambda xs, k: max(x[k] for x in xs)   # noqa: E731
    clock_ghz = 2.4
    return {
        "mfma_bf16": {"measured_tflops": best(mfma, "tflops"), "vendor_tflops": BF16_MFMA_PEAK_TFLOPS,
                      "runs": mfma, "note": "4 independent 32x32x16 bf16 accumulator chains per wave, "
                                            "register operands (random bf16)"},
        "mfma_softmax": {"measured_tflops": best(mix, "tflops"), "vendor_tflops": BF16_MFMA_PEAK_TFLOPS,
                         "runs": mix, "note": "MFMA rate of half the waves of each SIMD while the other half "
                                              "run the sweeps' softmax updates (FMA, v_exp_f32, add) in the "
                                              "sweeps' ratio: one update per lane per 256 MFMA flops"},
        "exp": {"measured_t_per_s": best(exps, "t_exp_per_s"), "derived_t_per_s": EXP_PEAK_T_PER_S,
                "runs": exps, "note": f"v_exp_f32, 8 independent chains per lane; derived figure = "
                                      f"half rate (8 lanes/clk/SIMD) x 4 SIMD x {cus} CU x {clock_ghz} GHz"},
        "hbm_copy": {"measured_gbs": best(copies, "gbs"), "vendor_gbs": HBM_PEAK_GBS, "bytes": 2 * nbytes,
                     "runs": copies, "note": "1 GiB read + 1 GiB written, 16-byte loads and stores"},
        "hbm_read": {"measured_gbs": best(reads, "gbs"), "vendor_gbs": HBM_PEAK_GBS, "bytes": rbytes,
                     "runs": reads, "note": "4 GiB read only, 16-byte loads, 8 in flight per thread"},
        "compute_units": cus,
    }


# ---------------------------------------------------------------- the whole stack (the headline)
def bench_stack(args, spec: syn.ConfigSpec, cpu) -> dict:
    """Every layer of a stack workload: the prompt phase (profile + compaction refilling each
    layer's cache) over all layers, then the decode loop, each generated token decoded through
    every layer's cache in turn.  Inputs are drawn on the device before timing starts."""
    import torch
    from adaptive_kv_cache_fg_amd import fastgen as fg
    from synth import device as sdev

    T = float(args.T) if args.T is not None else spec.T[0]
    L = spec.layers if args.stack_layers is None else args.stack_layers
    steps_dec = spec.decode_steps if args.decode_steps is None else args.decode_steps
    B, Hq, Hkv, n, d = spec.batch, spec.n_q_heads, spec.n_kv_heads, spec.seq_len, spec.head_dim
    G = Hq // Hkv
    e = 2 if spec.dtype == "bf16" else 4
    pool_n = min(16, steps_dec)
    dev = torch.device("cuda")
    say = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)   # noqa: E731

    # ---- inputs, resident in HBM before any timing
    t0 = time.perf_counter()
    lay = [sdev.make_layer_device(spec, l, dev) for l in range(L)]
    cls = lay[0].token_class                                   # classes depend on the batch entry only
    ncls_h = np.ascontiguousarray(np.stack([syn.new_token_classes(spec, b, steps_dec) for b in range(B)], axis=1))
    ncls = torch.from_numpy(ncls_h).to(dev)                    # [steps, B]
    pools = [sdev.make_decode_stream_device(spec, l, pool_n, dev, classes=ncls_h[:pool_n]) for l in range(L)]
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    say(f"inputs drawn on the device in {gen_s:.1f} s ({L} layers)")
    mk = int(max(np.count_nonzero(ncls_h[:, b]) for b in range(B)))
    outs = torch.empty((L, B, Hq, d), dtype=torch.float32, device=dev)
    caches = [None] * L
    profs = [None] * L

    profile_fn = fg.profile_rows if args.route == "rows" else fg.profile

    def prompt_phase(check=True):
        for l in range(L):
            c = caches[l]
            prof = profile_fn(lay[l].Q, lay[l].K, cls, spec.r_l, spec.r_f, T,
                              policy_out=None if c is None else c.t["policy"])
            caches[l] = fg.compact(lay[l].K, lay[l].V, cls, prof, Hq, max_new_tokens=steps_dec, max_new_kept=mk,
                                   reuse=c, check=check)
            profs[l] = prof

    def decode_tokens(t_a, t_b):
        for t in range(t_a, t_b):
            i = t % pool_n
            nc = ncls[t]
            for l in range(L):
                pl = pools[l]
                caches[l].decode_step(pl.q[i], pl.k[i], pl.v[i], nc, out=outs[l])

    # ---- first pass: allocates every cache (one read of the plan's totals per layer)
    t0 = time.perf_counter()
    prompt_phase()
    decode_tokens(0, min(2, steps_dec))
    torch.cuda.synchronize()
    say(f"caches allocated in {time.perf_counter() - t0:.1f} s; cache rows "
        f"{sum(int(c.c.total_rows) for c in caches)}")

    graphs = []
    pgraph = None
    mempool = None
    profs_graph = None
    if args.mode == "graph":
        # the prompt phase as one graph; the decode loop as graphs of --graph-tokens tokens each
        # (a decode step's position is a launch argument, so every graph covers its own tokens)
        t0 = time.perf_counter()
        mempool = torch.cuda.graph_pool_handle()
        pgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pgraph, pool=mempool):
            prompt_phase(check=False)
        profs_graph = list(profs)                              # the profiles the prompt graph writes
        prompt_phase()                                         # eager: host positions back to n
        torch.cuda.synchronize()
        for t_a in range(0, steps_dec, args.graph_tokens):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, pool=mempool):
                decode_tokens(t_a, min(steps_dec, t_a + args.graph_tokens))
            graphs.append(g)
        torch.cuda.synchronize()
        say(f"captured the prompt phase and {len(graphs)} decode graphs in {time.perf_counter() - t0:.1f} s")

    def one_step(ev=None):
        if ev is not None:
            ev[0].record()
        if pgraph is not None:
            pgraph.replay()
        else:
            prompt_phase(check=False)
        if ev is not None:
            ev[1].record()
        if graphs:
            for g in graphs:
                g.replay()
        else:
            decode_tokens(0, steps_dec)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    # correctness guard on the timed configuration: one step as timed, then the same step eagerly
    # with the plan's totals checked; outputs of the last token, the final caches' positions and the
    # profiles must agree bit for bit, and no cache may report an error
    one_step()
    torch.cuda.synchronize()
    ref_out = outs.clone()
    ref_state = [(c.t["pos"].clone(), c.t["len"].clone()) for c in caches]
    ref_prof = [(p.policy.clone(), p.recovery.clone(), p.cum.clone()) for p in (profs_graph if pgraph else profs)]
    # the check starts from caches whose rows are all NaN before the refill, so a row the refill or
    # a decode step should write and does not shows up in the outputs (the timed run's stale rows
    # hold the same stream's earlier values and would hide it)
    for c in caches:
        c.t["k"].fill_(float("nan"))
        c.t["v"].fill_(float("nan"))
    prompt_phase(check=True)
    for t_a in range(0, steps_dec, 256):
        decode_tokens(t_a, min(steps_dec, t_a + 256))
        torch.cuda.synchronize()
        say(f"eager check: {min(steps_dec, t_a + 256)} of {steps_dec} tokens")
    if not torch.equal(ref_out, outs):
        bad = [l for l in range(L) if not torch.equal(ref_out[l], outs[l])]
        raise RuntimeError(f"timed decode and eager decode disagree in layers {bad[:16]} ({len(bad)} of {L}); "
                           f"max |diff| {float((ref_out - outs).abs().max()):.3e}")
    for l in range(L):
        if not (torch.equal(ref_state[l][0], caches[l].t["pos"]) and torch.equal(ref_state[l][1], caches[l].t["len"])):
            raise RuntimeError(f"layer {l}: caches after the timed and the eager decode disagree")
        if not all(torch.equal(a, b) for a, b in zip(ref_prof[l], (profs[l].policy, profs[l].recovery, profs[l].cum))):
            raise RuntimeError(f"layer {l}: timed and eager prompt phases disagree")
        if caches[l].error_bits() != 0:
            raise RuntimeError(f"layer {l}: cache error bits set")
    del ref_out, ref_state, ref_prof
    say("timed configuration equals an eager run; timing")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        one_step(evs[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prompt_ms = float(np.median([ev[0].elapsed_time(ev[1]) for ev in evs]))   # median over the timed steps
    decode_ms = float(np.median([ev[1].elapsed_time(ev[2]) for ev in evs]))
    ms_per_step = wall * 1e3 / args.steps
    prompt_tok_s = B * n / (prompt_ms * 1e-3)
    decode_tok_s = B * steps_dec / (decode_ms * 1e-3)
    say(f"prompt {prompt_ms:.2f} ms ({prompt_tok_s:.4g} tok/s), decode {decode_ms:.1f} ms ({decode_tok_s:.4g} tok/s)")

    # ---- per-kernel figures (outside the timed region)
    # prompt kernels: one eager prompt phase with the library's events around every launch
    torch.cuda.synchronize()
    fg.timing_read()
    fg.timing_enable(True)
    prompt_phase(check=False)
    torch.cuda.synchronize()
    fg.timing_enable(False)
    per = {}
    for name, ms in fg.timing_read():
        per.setdefault(name, []).append(ms)
    kstats = {k: {"launches_per_step": float(len(v)), "avg_us": 1e3 * float(np.mean(v)),
                  "total_us_per_step": 1e3 * float(np.sum(v)), "timing": "events around each launch (eager pass)"}
              for k, v in per.items()}
    row_route = None
    if args.route == "columns" and not args.no_row_route:
        # the other recovery route (per-row level bins, fg_profile_rows) on every layer, one eager pass
        # with events around each launch; the cache refill is not needed for its cost
        fg.timing_read()
        fg.timing_enable(True)
        for l in range(L):
            fg.profile_rows(lay[l].Q, lay[l].K, cls, spec.r_l, spec.r_f, T)
        torch.cuda.synchronize()
        fg.timing_enable(False)
        rr = {}
        for name, ms in fg.timing_read():
            rr.setdefault(name, []).append(ms)
        row_route = {k: {"avg_us": 1e3 * float(np.mean(v)), "launches": len(v)} for k, v in rr.items()}

    def rows_kept(c):
        """Cache rows in use that hold a key (pos >= 0), summed over the heads of one layer."""
        total = int(c.c.total_rows)
        ro = c.t["row_offset"]
        idx = torch.arange(total, device=dev, dtype=torch.int64)
        head = torch.bucketize(idx, ro[1:], right=True).clamp_(max=ro.numel() - 2)
        in_use = idx < ro[head] + c.t["len"].to(torch.int64)[head]
        return int((in_use & (c.t["pos"][:total] >= 0)).sum().item())

    def partials_graph_us(reps):
        """fg_decode_partials (the split-K launch alone, read-only on the caches) for every layer,
        captured as a graph of `reps` passes over the layers; events around its replay (eager
        mode: the same launches from Python, events around the loop)."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        if args.mode == "eager":
            for l in range(L):
                caches[l].decode_partials(pools[l].q[0])
            torch.cuda.synchronize()
            ev[0].record()
            for r in range(reps):
                for l in range(L):
                    caches[l].decode_partials(pools[l].q[r % pool_n])
            ev[1].record()
            torch.cuda.synchronize()
            return 1e3 * ev[0].elapsed_time(ev[1]) / (reps * L)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, pool=mempool):
            for r in range(reps):
                for l in range(L):
                    caches[l].decode_partials(pools[l].q[r % pool_n])
        g.replay()
        torch.cuda.synchronize()
        ev[0].record()
        g.replay()
        ev[1].record()
        torch.cuda.synchronize()
        del g
        return 1e3 * ev[0].elapsed_time(ev[1]) / (reps * L)

    # the split-K launch at the first and at the last decode state (rows grow linearly in between)
    prompt_phase(check=False)
    torch.cuda.synchronize()
    kept_start = [rows_kept(c) for c in caches]
    p_start = partials_graph_us(4)
    decode_tokens(0, steps_dec)
    torch.cuda.synchronize()
    kept_end = [rows_kept(c) for c in caches]
    p_end = partials_graph_us(4)
    q_bytes = B * Hq * d * e
    row_bytes = 2 * d * e + 4
    mean_rows = 0.5 * (sum(kept_start) + sum(kept_end)) / L          # per layer, mean over the steps
    part_bytes = mean_rows * row_bytes + q_bytes
    part_us = 0.5 * (p_start + p_end)
    step_us = 1e3 * decode_ms / (steps_dec * L)                       # one layer's decode step
    merge_us = step_us - part_us
    merge_bytes = B * Hkv * 2 * d * e + B * Hq * d * (e + 4)
    step_bytes = part_bytes + merge_bytes
    kstats["decode_partials"] = {
        "launches_per_step": float(steps_dec * L), "avg_us": part_us, "total_us_per_step": part_us * steps_dec * L,
        "timing": f"graphs of fg_decode_partials over every layer, events around the replay, at the first "
                  f"({p_start:.2f} us) and the last ({p_end:.2f} us) decode state; the mean"}
    kstats["decode_merge"] = {
        "launches_per_step": float(steps_dec * L), "avg_us": merge_us, "total_us_per_step": merge_us * steps_dec * L,
        "timing": "timed decode step minus the graph-timed split-K launch"}
    kstats["decode_step"] = {
        "launches_per_step": float(steps_dec * L), "avg_us": step_us, "total_us_per_step": 1e3 * decode_ms,
        "note": "one layer's whole decode step (both launches and the gaps between them), from the timed region"}

    # algorithmic work
    pairs = n * (n + 1) // 2
    sweep_flops = B * Hq * 2 * d * pairs                              # per sweep launch (one layer)
    sweep_exps = B * Hq * pairs
    kept_prompt = [c.kept_count.to(torch.int64).sum().item() for c in caches]   # prompt keys kept per layer
    gather_bytes = float(np.mean([k * (2 * 2 * d * e + 4) for k in kept_prompt])) + B * Hkv * (n + n / 8)
    peak_mfma = BF16_MFMA_PEAK_TFLOPS if spec.dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS
    for k, units, bound in (("profile_rowstats", sweep_flops, "mfma"), ("profile_colsums", sweep_flops, "mfma"),
                            ("compact_gather", gather_bytes, "hbm"), ("decode_partials", part_bytes, "hbm"),
                            ("decode_merge", merge_bytes, "hbm"), ("decode_step", step_bytes, "hbm")):
        if k not in kstats:
            continue
        avg_s = kstats[k]["avg_us"] * 1e-6
        if bound == "mfma":
            ach = units / avg_s / 1e12
            kstats[k].update(bound="mfma", achieved=ach, peak=peak_mfma, unit="TFLOP/s", frac=ach / peak_mfma,
                             algorithmic_flops=units, exps=sweep_exps,
                             exp_rate_t_per_s=sweep_exps / avg_s / 1e12,
                             exp_frac=sweep_exps / avg_s / 1e12 / EXP_PEAK_T_PER_S)
        else:
            ach = units / avg_s / 1e9
            kstats[k].update(bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s", frac=ach / HBM_PEAK_GBS,
                             algorithmic_bytes=units)
    if row_route is not None:
        rb = row_route.get("profile_rowbins")
        if rb:
            ach = sweep_flops / (rb["avg_us"] * 1e-6) / 1e12
            rb.update(bound="mfma", achieved=ach, peak=peak_mfma, unit="TFLOP/s", frac=ach / peak_mfma,
                      note="score flops only (the binning products add half as many again)")
        per_layer = sum(v["avg_us"] * v["launches"] for v in row_route.values()) / L
        cols_layer = sum(kstats[k]["total_us_per_step"] for k in ("profile_rowstats", "profile_colsums",
                                                                   "profile_select") if k in kstats) / L
        row_route = {"kernels": row_route, "profile_rows_us_per_layer": per_layer,
                     "profile_columns_us_per_layer": cols_layer,
                     "note": "fg_profile_rows (recovery from the per-row level bins, plus the least kept share "
                             "of any row) against fg_profile (recovery from the column sums), events around each "
                             "launch, every layer; bench.py --route rows times the prompt phase with it"}
    dominant = max((k for k in ("profile_rowstats", "profile_colsums", "compact_gather", "decode_partials",
                                "decode_merge") if k in kstats), key=lambda k: kstats[k]["total_us_per_step"])
    dk = kstats[dominant]
    key = stack_workload_key(spec, T, L, steps_dec)
    roofline = {"bound": dk["bound"], "achieved": dk["achieved"], "peak": dk["peak"], "unit": dk["unit"],
                "frac": dk["frac"], "traffic": measured_traffic(dominant, key), "kernel": dominant}

    # the whole phases against their ceilings
    prompt_flops = 2 * sweep_flops * L
    decode_bytes = step_bytes * L * steps_dec
    phases = {
        "prompt_mfma_frac": prompt_flops / (prompt_ms * 1e-3) / 1e12 / peak_mfma,
        "prompt_flops": prompt_flops,
        "decode_hbm_frac": decode_bytes / (decode_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "decode_bytes": decode_bytes,
        "decode_cache_bytes_per_token": mean_rows * row_bytes * L,
        "note": "prompt: both sweeps' algorithmic flops over every layer / prompt-phase time (profile, select, "
                "plan, gather included); decode: algorithmic bytes of every layer's steps (cache rows kept, "
                "mean of the first and last state; q, new k/v, fp32 output) / decode time",
    }
    pol = np.concatenate([p.policy.cpu().numpy().reshape(-1) for p in profs])
    full_rows = B * Hkv * (n + (steps_dec - 1) / 2.0) * L
    compression = {
        "policy_histogram": np.bincount(pol, minlength=5).tolist(),
        "prompt_keys_kept_fraction": float(sum(kept_prompt) / (B * Hkv * n * L)),
        "kv_bytes_full_per_token": full_rows * 2 * d * e,
        "kv_bytes_adaptive_per_token": mean_rows * L * 2 * d * e,
        "kv_pruned_fraction": 1.0 - mean_rows * L / full_rows,
        "note": "KV bytes a decode step reads, mean over the steps: every key kept (full) vs the adaptive caches",
    }
    pk = None
    if not args.no_peaks:
        pk = chip_peaks(torch, fg)
        mf, ex, cp = pk["mfma_bf16"]["measured_tflops"], pk["exp"]["measured_t_per_s"], pk["hbm_copy"]["measured_gbs"]
        rd = pk["hbm_read"]["measured_gbs"]
        for k in ("profile_rowstats", "profile_colsums"):
            if k in kstats:
                kstats[k]["frac_of_measured_mfma"] = kstats[k]["achieved"] / mf
                kstats[k]["exp_frac_of_measured"] = kstats[k]["exp_rate_t_per_s"] / ex
                kstats[k]["frac_of_measured_mfma_softmax"] = kstats[k]["achieved"] / pk["mfma_softmax"]["measured_tflops"]
        for k in ("compact_gather", "decode_partials", "decode_step"):
            kstats[k]["frac_of_measured_copy"] = kstats[k]["achieved"] / cp
        for k in ("decode_partials", "decode_step"):                 # read streams: the read ceiling
            kstats[k]["frac_of_measured_read"] = kstats[k]["achieved"] / rd
        phases["prompt_frac_of_measured_mfma"] = phases["prompt_mfma_frac"] * peak_mfma / mf
        phases["prompt_frac_of_measured_mfma_softmax"] = (phases["prompt_mfma_frac"] * peak_mfma /
                                                          pk["mfma_softmax"]["measured_tflops"])
        phases["decode_frac_of_measured_copy"] = phases["decode_hbm_frac"] * HBM_PEAK_GBS / cp
        phases["decode_frac_of_measured_read"] = phases["decode_hbm_frac"] * HBM_PEAK_GBS / rd
        ceiling = mf if dk["bound"] != "hbm" else (rd if dominant.startswith("decode") else cp)
        roofline["frac_of_measured"] = dk["achieved"] / ceiling
        roofline["measured_ceiling"] = {"value": ceiling, "unit": dk["unit"],
                                        "kind": "mfma" if dk["bound"] != "hbm" else
                                        ("hbm_read" if dominant.startswith("decode") else "hbm_copy")}

    calibration_copy(torch, fg)

    workload = (f"{spec.name}: {L} layers x {Hq} heads (KV {Hkv}), d={d}, {spec.dtype}, B={B}, n={n}, "
                f"T={T}, r_l={spec.r_l}, r_f={spec.r_f}, {steps_dec} decode steps through every layer")
    return {
        "metric": METRIC, "value": prompt_tok_s, "unit": "prompt tok/s (profile+compact)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype,
        "data": "synthetic (seeded Llama-shaped post-RoPE Q/K/V with planted head types, drawn on the device)",
        "config": {"workload": workload, "layers": L, "batch": B, "seq_len": n, "decode_steps": steps_dec, "T": T,
                   "key": key},
        "decode_tok_s": decode_tok_s, "mode": args.mode, "prompt_ms": prompt_ms, "decode_ms": decode_ms,
        "roofline": roofline, "phases": phases, "compression": compression, "kernels": kstats,
        "route": args.route, "row_route": row_route,
        "peaks": pk, "input_generation_s": gen_s, "cpu_baseline": cpu,
    }


# ---------------------------------------------------------------- rocprofv3 summaries
def _csv_rows(directory: str, suffix: str):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


def _short(name: str) -> str:
    """Kernel name without namespace, template arguments and parameter list (mangled or not)."""
    if name.startswith("_ZN"):                           # Itanium mangling: _ZN <len><id> ... then I / E
        i, parts = 3, []
        while i < len(name) and name[i].isdigit():
            j = i
            while name[j].isdigit():
                j += 1
            k = int(name[i:j])
            parts.append(name[j:j + k])
            i = j + k
        if parts:
            return parts[-1]
    base = name.split("(")[0]
    depth, out = 0, []
    for ch in base:
        depth += ch == "<"
        if depth == 0:
            out.append(ch)
        depth -= ch == ">"
    s = "".join(out).strip()
    return s.split("::")[-1].split(" ")[-1] or name[:48]


def summarize_trace(directory: str, title: str, command: str) -> str:
    """Text summary of a rocprofv3 --kernel-trace --stats run: per kernel, calls and average /
    min / max dispatch durations from the kernel trace."""
    trace = _csv_rows(directory, "kernel_trace.csv")
    per = {}
    for r in trace:
        name = _short(r.get("Kernel_Name", ""))
        t = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per.setdefault(name, []).append(t)
    total = sum(sum(v) for v in per.values()) or 1.0
    lines = [f"# {title}", f"# command: {command}",
             "# durations in microseconds per dispatch (profiler timestamps), from the kernel trace",
             f"{'kernel':44s} {'calls':>8s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{name[:44]:44s} {len(v):8d} {np.mean(v):9.2f} {np.min(v):9.2f} {np.max(v):9.2f} "
                     f"{100 * sum(v) / total:6.2f}")
    return "\n".join(lines) + "\n"


def _counter_means(directory: str, counter: str) -> dict:
    """Mean of one counter per dispatch, by short kernel name (rocprofv3 --pmc counter collection);
    the calibration copy (peak_copy_kernel launched with CALIB_BLOCKS workgroups) under its own key."""
    per = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        k = _short(r.get("Kernel_Name", ""))
        if k == "peak_copy_kernel" and int(float(r.get("Grid_Size", 0))) == CALIB_BLOCKS * 256:
            k = "calibration_copy"
        per.setdefault(k, []).append(float(r["Counter_Value"]))
    return {k: (float(np.mean(v)), len(v)) for k, v in per.items()}


def summarize_counters(directories, title: str, command: str) -> str:
    """Per library kernel, the mean per dispatch of every counter in rocprofv3 --pmc runs."""
    per = {}
    for directory in directories:
        for r in _csv_rows(directory, "counter_collection.csv"):
            k = _short(r.get("Kernel_Name", ""))
            per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    names = sorted({c for v in per.values() for c in v})
    lines = [f"# {title}", f"# commands: {command}", "# mean per dispatch over the dispatches of the run",
             f"{'kernel':28s} {'dispatches':>10s} " + " ".join(f"{c:>22s}" for c in names)]
    for k, v in sorted(per.items()):
        if not k.endswith("_kernel") or k.startswith(("elementwise", "vectorized")):
            continue
        cnt = max(len(x) for x in v.values())
        lines.append(f"{k[:28]:28s} {cnt:10d} " + " ".join(
            f"{np.mean(v[c]):22.4g}" if c in v else f"{'-':>22s}" for c in names))
    return "\n".join(lines) + "\n"


def record_traffic(fetch_dir: str, write_dir: str, key: str, command: str) -> str:
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what they read for the 256 MiB copy
    the benchmark issues after its timed region, store the per-launch bytes of the library's
    kernels in profiles/traffic.json under ``key`` with the current sources' digest, and return
    a text summary."""
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    calib = "calibration_copy"
    f_factor = CALIB_BYTES / (fetch[calib][0] * 1024)
    w_factor = CALIB_BYTES / (write[calib][0] * 1024)
    names = {"rowstats_kernel": "profile_rowstats", "colsums_kernel": "profile_colsums",
             "gather_kernel": "compact_gather", "decode_partials_kernel": "decode_partials",
             "decode_merge_kernel": "decode_merge", "select_kernel": "profile_select"}
    per_launch = {}
    lines = [f"# HBM traffic per dispatch, {key}", f"# commands: {command}",
             "# FETCH_SIZE / WRITE_SIZE: rocprofv3 derived counters in KiB per dispatch, averaged over dispatches;",
             f"# scaled bytes = FETCH * {f_factor:.4f} + WRITE * {w_factor:.4f} (factors from the {CALIB_BYTES} B "
             f"calibration copy: FETCH {fetch[calib][0]:.1f} KiB, WRITE {write[calib][0]:.1f} KiB)"]
    for k, short in names.items():
        if k not in fetch or k not in write:
            continue
        (fv, nf), (wv, _) = fetch[k], write[k]
        b = fv * 1024 * f_factor + wv * 1024 * w_factor
        per_launch[short] = b
        lines.append(f"{k:26s} dispatches {nf:7d}  FETCH_SIZE {fv:13.1f} KiB  WRITE_SIZE {wv:12.1f} KiB  "
                     f"scaled bytes {b:14.0f}")
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        t = {}
    t = {"workloads": t.get("workloads", {})}
    t["workloads"][key] = {"sources_digest": {k: kernel_sources_digest(k) for k in per_launch},
                           "fetch_factor": f_factor, "write_factor": w_factor, "bytes_per_launch": per_launch}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
    return "\n".join(lines) + "\n"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=3,
                    help="workload id (3 = the Llama-1-65B-shaped stack, the default; 1 = one Llama-1-7B layer)")
    ap.add_argument("--layer", type=int, default=None,
                    help="one layer of a stack workload instead of the whole stack")
    ap.add_argument("--T", type=float, default=None, help="recover ratio (default: the workload's first)")
    ap.add_argument("--stack-layers", type=int, default=None, help=argparse.SUPPRESS)
    ap.add_argument("--decode-steps", type=int, default=None, help=argparse.SUPPRESS)
    ap.add_argument("--graph-tokens", type=int, default=16, help="generated tokens per captured decode graph")
    ap.add_argument("--route", choices=["columns", "rows"], default="columns",
                    help="recovery route of the prompt phase: column sums (fg_profile) or per-row level bins "
                         "(fg_profile_rows)")
    ap.add_argument("--no-row-route", action="store_true", help="skip timing the per-row route beside the default")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the Llama-1-7B-shaped stack at its three T after the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-heads", type=int, default=16)
    ap.add_argument("--cpu-only", action="store_true",
                    help="time only the CPU oracle (every KV head of a one-layer workload; the sampled layers "
                         "of a stack) and exit")
    ap.add_argument("--no-peaks", action="store_true", help="skip the chip-ceiling micro-benchmarks")
    ap.add_argument("--no-full-baseline", action="store_true",
                    help="one layer: skip the full-cache decode baseline (every head keeps every key)")
    ap.add_argument("--no-attention", action="store_true",
                    help="one layer: skip the prompt-attention measurement")
    ap.add_argument("--no-stability", action="store_true",
                    help="one layer: skip the decode-time stability measurement over full caches")
    ap.add_argument("--mode", "--decode-mode", dest="mode", choices=["graph", "eager"], default="graph",
                    help="graph: the prompt phase and the decode loop captured as HIP graphs and replayed; "
                         "eager: every call launched from Python")
    ap.add_argument("--summarize-trace", metavar="DIR", default=None,
                    help="print a summary of a rocprofv3 --kernel-trace run's output directory and exit")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="scale two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into profiles/traffic.json "
                         "under --key, print the summary and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR", default=None,
                    help="print per-kernel counter means of rocprofv3 --pmc runs and exit")
    ap.add_argument("--key", default=None, help="workload key for --record-traffic")
    ap.add_argument("--title", default="", help="title line of --summarize-trace")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.title, args.command), end="")
        return 0
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.title, args.command), end="")
        return 0
    if args.record_traffic:
        print(record_traffic(args.record_traffic[0], args.record_traffic[1], args.key, args.command), end="")
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU (each box has one); --gpus must be 1. The path "
                                   "shards by (batch entry, layer, KV head) with no exchange between GPUs."}))
        return 2
    spec = syn.CONFIGS[args.config]
    stack = spec.layers > 1 and args.layer is None
    if not stack:
        args.layer = 0 if args.layer is None else args.layer
        if not 0 <= args.layer < spec.layers:
            print(json.dumps({"error": f"--layer must be in [0, {spec.layers})"}))
            return 2
    if args.cpu_only:
        # the oracle alone: every KV head of a one-layer workload, or the stack's sampled layers
        cpu = (cpu_baseline_stack(spec, spec.layers) if spec.layers > 1 else
               cpu_baseline(spec, spec.n_kv_heads, 0))
        print(json.dumps({"config": spec.name, "cpu_baseline": cpu}))
        return 0
    cpu = None
    if not args.no_cpu_baseline:                              # before any GPU call (fork pool)
        if stack:
            cpu = cpu_baseline_stack(spec, spec.layers if args.stack_layers is None else args.stack_layers)
        else:
            cpu = cpu_baseline(spec, args.cpu_sample_heads, args.layer)
    result = bench_stack(args, spec, cpu) if stack else bench_layer(args, spec, cpu)
    if stack and args.config == 3 and args.stack_layers is None and not args.no_secondary:
        result["secondary"] = secondary_llama7b_stack(args)
    print(json.dumps(result))
    return 0


def secondary_llama7b_stack(args) -> dict:
    """The Llama-1-7B-shaped stack (32 layers x 32 heads, B=8, n=4096, 512 decode steps) at each of
    its three T, outside the headline's timing: 2 timed steps after 1 warm-up each."""
    import copy
    import gc
    import torch
    gc.collect()
    torch.cuda.empty_cache()
    spec = syn.CONFIGS[2]
    out = {}
    for T in spec.T:
        a = copy.copy(args)
        a.steps, a.warmup, a.T = 2, 1, T
        a.no_peaks = True
        a.no_row_route = True
        r = bench_stack(a, spec, None)
        out[f"T={T}"] = {
            "prompt_tok_s": r["value"], "decode_tok_s": r["decode_tok_s"], "prompt_ms": r["prompt_ms"],
            "decode_ms": r["decode_ms"], "prompt_mfma_frac": r["phases"]["prompt_mfma_frac"],
            "decode_hbm_frac": r["phases"]["decode_hbm_frac"],
            "decode_partials_hbm_frac": r["kernels"]["decode_partials"]["frac"],
            "policy_histogram": r["compression"]["policy_histogram"],
            "kv_pruned_fraction": r["compression"]["kv_pruned_fraction"],
            "prompt_keys_kept_fraction": r["compression"]["prompt_keys_kept_fraction"],
        }
        gc.collect()
        torch.cuda.empty_cache()
    return {"workload": f"{spec.name}: {spec.layers} layers x {spec.n_q_heads} heads, d={spec.head_dim}, "
                        f"{spec.dtype}, B={spec.batch}, n={spec.seq_len}, r_l={spec.r_l}, r_f={spec.r_f}, "
                        f"{spec.decode_steps} decode steps through every layer",
            "per_T": out, "note": "the same measurement as the headline, 2 timed steps after 1 warm-up per T"}


if __name__ == "__main__":
    sys.exit(main())
