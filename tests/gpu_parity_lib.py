"""Shared machinery of the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, run the oracle on the same inputs, compare.

Tolerances (fixed by the parity contract, written once here):
* kept-index lists, frequent sets, policies: exact, except heads the oracle
  flags -- a recovery within 1e-4 of T (near-T) or a k-th cumulative score whose
  relative gap to the next is below TIE_TAU (top-k tie); flagged heads get the
  weaker checks below and the downstream steps run in forced mode (the oracle
  takes the GPU's policy and frequent set);
* recovery: 1e-4 absolute;
* decode outputs: max |gpu - oracle| <= 2e-3 * max |oracle| per output vector for
  bf16 inputs, 1e-5 for fp32;
* the cache after every decode step: the exact set of kept positions;
* prompt attention output O (bf16): per element
  |gpu - oracle| <= (2^-8 + 5e-4) * (A|V|)_i + 2^-8 * |O_i|, from the bf16
  rounding of the softmax numerators fed to the P V product (unit roundoff
  2^-8 on each term), the bf16 rounding of the output, and fp32 slack for the
  score and sum accumulation; plus an RMS of the normalised error <= 2^-9.
"""
from __future__ import annotations

import math
import sys
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from adaptive_kv_cache_fg_amd import fastgen as fg
from oracle import fastgen_ref as ref
from synth import inputs as syn

TIE_TAU = 3e-5
REC_TOL = 1e-4
DEC_TOL = {"bf16": 2e-3, "f32": 1e-5}


def upload(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        bits = syn.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@dataclass
class HeadReport:
    b: int
    h: int
    kind: str
    policy_gpu: int
    policy_ref: int
    near_T: bool
    topk_tie: bool
    rec_err: float
    cum_rel_err: float
    lse_err: float


@dataclass
class CaseReport:
    heads: List[HeadReport] = field(default_factory=list)
    dec_err: float = 0.0
    flagged: int = 0


def allowed_policies(R: np.ndarray, T: float, ref_policy: int) -> set:
    ok = {ref_policy}
    for k in range(4):
        if abs(R[k] - T) <= ref.NEAR_T_WINDOW:
            ok.add(k)
            ok.add(k + 1)
    return ok


def eps_topk_ok(cum_ref: np.ndarray, F_gpu: np.ndarray, k_f: int, tau: float) -> bool:
    """Every chosen key scores at least the k-th minus the window, every rejected one at most
    the (k+1)-th plus the window (oracle scores)."""
    if F_gpu.sum() != min(max(k_f, 0), len(cum_ref)):
        return False
    if k_f <= 0 or k_f >= len(cum_ref):
        return True
    s = np.sort(cum_ref)[::-1]
    sk, sk1 = s[k_f - 1], s[k_f]
    w = tau * sk + 2.0 ** -100
    return bool(np.all(cum_ref[F_gpu] >= sk - w) and np.all(cum_ref[~F_gpu] <= sk1 + w))


def download(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def check_attention_head(O_g: np.ndarray, Qg: np.ndarray, K: np.ndarray, V: np.ndarray,
                         rows: Optional[np.ndarray] = None) -> float:
    """O_g [G, n, d] (or [G, len(rows), d]) of one KV head against the oracle; returns the
    largest error relative to the bound."""
    if rows is None:
        want = ref.attention_output(Qg, K, V)
        scale = ref.attention_output(Qg, K, np.abs(V))
    else:
        G = Qg.shape[0]
        want = np.empty((G, len(rows), V.shape[1]))
        scale = np.empty_like(want)
        for g in range(G):
            for k, r in enumerate(rows):
                a = ref.causal_attention_rows(Qg[g, r:r + 1], K[: r + 1], int(r))
                want[g, k] = (a @ V[: r + 1])[0]
                scale[g, k] = (a @ np.abs(V[: r + 1]))[0]
    err = np.abs(O_g - want)
    bound = (2.0 ** -8 + 5e-4) * scale + 2.0 ** -8 * np.abs(want)
    worst = float(np.max(err / bound))
    assert worst <= 1.0, ("attention output outside the rounding bound", worst)
    rms = float(np.sqrt(np.mean((err / (scale + np.abs(want))) ** 2)))
    assert rms <= 2.0 ** -9, ("attention output error not rounding-sized", rms)
    return worst


def run_case(spec: syn.ConfigSpec, layer: int = 0, T: Optional[float] = None, steps: Optional[int] = None,
             batch=None, seed=None, check_decode: bool = True, fused: bool = False) -> CaseReport:
    T = spec.T[0] if T is None else T
    steps = spec.decode_steps if steps is None else steps
    log(f"[case] cfg={spec.cfg_id} {spec.name} B={spec.batch} Hq={spec.n_q_heads} Hkv={spec.n_kv_heads} "
        f"n={spec.seq_len} d={spec.head_dim} {spec.dtype} T={T} steps={steps}")
    li = syn.make_layer(spec, layer, batch=batch, seed=seed)
    B, Hq, n, d = li.Q.shape
    Hkv = li.K.shape[1]
    G = Hq // Hkv
    Qd, Kd, Vd = upload(li.Q, spec.dtype), upload(li.K, spec.dtype), upload(li.V, spec.dtype)
    cls_d = torch.from_numpy(li.token_class).cuda()
    prof = fg.profile(Qd, Kd, cls_d, spec.r_l, spec.r_f, T, want_lse=True, want_band=True,
                      V=Vd if fused else None)
    torch.cuda.synchronize()
    if fused:                                  # the attention output the profiling rode on
        O_g = download(prof.out)
        for b in range(B):
            for h in range(Hkv):
                check_attention_head(O_g[b, h * G:(h + 1) * G], li.Q[b, h * G:(h + 1) * G].astype(np.float64),
                                     li.K[b, h].astype(np.float64), li.V[b, h].astype(np.float64))
    pol_g = prof.policy.cpu().numpy()
    cum_g = prof.cum.cpu().numpy().astype(np.float64)
    band_g = prof.band.cpu().numpy().astype(np.float64)
    lse_g = prof.lse.cpu().numpy().astype(np.float64)
    rec_g = prof.recovery.cpu().numpy().astype(np.float64)
    F_g = prof.frequent()
    rep = CaseReport()
    forced = {}
    for b in range(B):
        for h in range(Hkv):
            pr = ref.profile_head(li.Q[b, h * G:(h + 1) * G], li.K[b, h], li.token_class[b], spec.r_l, spec.r_f, T,
                                  tau=TIE_TAU)
            lse_err = float(np.max(np.abs(lse_g[b, h * G:(h + 1) * G] - pr.lse)))
            cum_rel = float(np.max(np.abs(cum_g[b, h] - pr.cum) / np.maximum(pr.cum, 1e-30)))
            rec_err = float(np.max(np.abs(rec_g[b, h] - pr.R)))
            # checks
            assert lse_err <= 2e-4 + 2e-6 * float(np.max(np.abs(pr.lse))), (b, h, lse_err)
            assert np.allclose(cum_g[b, h], pr.cum, rtol=2e-4, atol=1e-6 * G), (b, h, cum_rel)
            assert np.allclose(band_g[b, h], pr.band, rtol=2e-4, atol=1e-6 * G), (b, h)
            assert rec_err <= REC_TOL, (b, h, rec_g[b, h], pr.R)
            assert np.all(np.diff(rec_g[b, h]) >= -1e-6) and rec_g[b, h, 4] == 1.0
            if pr.topk_tie:
                assert eps_topk_ok(pr.cum, F_g[b, h], pr.k_f, TIE_TAU), (b, h)
            else:
                assert np.array_equal(F_g[b, h], pr.F), (b, h, np.flatnonzero(F_g[b, h] != pr.F)[:10])
            if pr.near_T or pr.topk_tie:
                rep.flagged += 1
                assert int(pol_g[b, h]) in allowed_policies(pr.R, T, pr.policy), (b, h)
            else:
                assert int(pol_g[b, h]) == pr.policy, (b, h, rec_g[b, h], pr.R)
            # the GPU's own decision follows from its own recovery values
            own = next(k for k in range(5) if rec_g[b, h, k] >= T or k == 4)
            if not np.any(np.abs(rec_g[b, h, :4] - T) < 1e-6):
                assert int(pol_g[b, h]) == own, (b, h, rec_g[b, h])
            forced[(b, h)] = (int(pol_g[b, h]), F_g[b, h].copy(), pr)
            rep.heads.append(HeadReport(b, h, li.types[h], int(pol_g[b, h]), pr.policy, pr.near_T, pr.topk_tie,
                                        rec_err, cum_rel, lse_err))
    max_new = steps
    cache = fg.compact(Kd, Vd, cls_d, prof, Hq, max_new_tokens=max_new, max_new_kept=max_new)
    kept_g = cache.kept_positions()
    for (b, h), (pol, Fg_, pr) in forced.items():
        want = ref.kept_positions(li.token_class[b], Fg_, pr.w_l, pol)
        assert np.array_equal(kept_g[b * Hkv + h], want), (b, h, pol)
        if pol == pr.policy and not pr.topk_tie:
            assert np.array_equal(want, pr.kept)
    # compacted bytes equal the source rows
    for hd in range(B * Hkv):
        pos, kc, vc = cache.rows(hd)
        sel = pos >= 0
        b, h = divmod(hd, Hkv)
        assert torch.equal(kc[torch.from_numpy(sel).cuda()], Kd[b, h][torch.from_numpy(pos[sel]).cuda().long()])
        assert torch.equal(vc[torch.from_numpy(sel).cuda()], Vd[b, h][torch.from_numpy(pos[sel]).cuda().long()])
    if not check_decode or steps == 0:
        return rep
    ds = syn.make_decode_stream(spec, layer, steps, batch=batch, seed=seed)
    outs = []
    caches = []
    for t in range(steps):
        q = upload(ds.q[t], spec.dtype)
        kn = upload(ds.k[t], spec.dtype)
        vn = upload(ds.v[t], spec.dtype)
        nc = torch.from_numpy(ds.new_class[t].copy()).cuda()
        outs.append(cache.decode_step(q, kn, vn, nc).cpu().numpy())
        if t < 8 or t == steps - 1 or t % 16 == 0:
            caches.append((t, cache.kept_positions()))
    assert cache.error_bits() == 0
    outs = np.stack(outs)                                   # [steps, B, Hq, d]
    tol = DEC_TOL[spec.dtype]
    worst = 0.0
    for (b, h), (pol, Fg_, pr) in forced.items():
        o_ref, c_ref = ref.decode_incremental(li.K[b, h], li.V[b, h], li.token_class[b], Fg_, pr.w_l, pol,
                                              ds.q[:, b, h * G:(h + 1) * G], ds.k[:, b, h], ds.v[:, b, h],
                                              ds.new_class[:, b])
        o_gpu = outs[:, b, h * G:(h + 1) * G]
        scale = np.maximum(np.max(np.abs(o_ref), axis=-1), 1e-30)
        err = np.max(np.abs(o_gpu - o_ref), axis=-1) / scale
        worst = max(worst, float(err.max()))
        assert err.max() <= tol, (b, h, pol, float(err.max()))
        for t, kept in caches:
            assert np.array_equal(kept[b * Hkv + h], c_ref[t]), (b, h, t)
    rep.dec_err = worst
    log(f"[case] ok: heads={len(rep.heads)} flagged={rep.flagged} "
        f"max rec err={max(x.rec_err for x in rep.heads):.2e} "
        f"max cum rel err={max(x.cum_rel_err for x in rep.heads):.2e} "
        f"max lse err={max(x.lse_err for x in rep.heads):.2e} dec err={worst:.2e} "
        f"policies={np.bincount([x.policy_gpu for x in rep.heads], minlength=5).tolist()}")
    return rep


# ---------------------------------------------------------------- full-size layers, sampled heads

def _oracle_heads(Qh, Kh, cls_h, spec, heads, T, tau=TIE_TAU):
    """Oracle profiles of the sampled (b, h) heads from host copies Qh [B, Hq, n, d] / Kh [B, Hkv, n, d]
    (only the sampled slices need to be filled).  Heads run on an outer thread pool, each head's row
    blocks on an inner one (numpy releases the GIL; BLAS limited to one thread per worker)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    G = spec.group
    workers = min(16, len(os.sched_getaffinity(0)))

    with threadpool_limits(1), ThreadPoolExecutor(max_workers=workers) as inner, \
            ThreadPoolExecutor(max_workers=max(1, workers // 2)) as outer:
        def one(bh):
            b, h = bh
            return bh, ref.profile_head(Qh[b, h * G:(h + 1) * G], Kh[b, h], cls_h[b], spec.r_l, spec.r_f, T,
                                        tau=tau, executor=inner)
        out = {}
        for k, (bh, pr) in enumerate(outer.map(one, heads)):
            out[bh] = pr
            if k % 16 == 15 or k == len(heads) - 1:
                log(f"[oracle] {k + 1} of {len(heads)} heads done")
    return out


class _oracle_pool:
    """A thread pool for per-head oracle work, BLAS limited to one thread per worker."""

    def __enter__(self):
        import os
        from concurrent.futures import ThreadPoolExecutor
        from threadpoolctl import threadpool_limits
        self._lim = threadpool_limits(1)
        self._ex = ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0))))
        return self._ex

    def __exit__(self, *exc):
        self._ex.shutdown()
        self._lim.restore_original_limits()
        return False


def run_fullsize(spec: syn.ConfigSpec, layer: int, sample: List[tuple], decode_sample: List[tuple],
                 Ts=None, steps: Optional[int] = None, out_steps: Optional[List[int]] = None) -> dict:
    """One full-size layer drawn on the device (synth.device), every T of the workload:
    * every head: column sums total G n, recovery monotone with R_4 = 1, |F| = k_f, the policy the
      GPU's own recovery implies, the kept list under the GPU's policy and frequent set, and the
      cache after the last decode step (positions, exact);
    * the sampled heads against the oracle: lse, cum, band, recovery (1e-4), frequent set and
      policy (exact unless flagged), compacted bytes;
    * decode outputs of the decode-sampled heads at every step in ``out_steps`` (default: all)."""
    from synth import device as sdev
    Ts = list(spec.T) if Ts is None else list(Ts)
    steps = spec.decode_steps if steps is None else steps
    out_steps = list(range(steps)) if out_steps is None else sorted(set(out_steps))
    log(f"[fullsize] cfg={spec.cfg_id} {spec.name} layer={layer} B={spec.batch} Hq={spec.n_q_heads} "
        f"Hkv={spec.n_kv_heads} n={spec.seq_len} T={Ts} steps={steps} sample={len(sample)} "
        f"decode sample={len(decode_sample)} output steps={len(out_steps)}")
    li = sdev.make_layer_device(spec, layer, "cuda")
    Qd, Kd, Vd, cls_d = li.Q, li.K, li.V, li.token_class
    B, Hq, n, d = Qd.shape
    Hkv = Kd.shape[1]
    G = Hq // Hkv
    cls_h = li.token_class_host
    Kh = sdev.host_f32(Kd)
    Vh = sdev.host_f32(Vd)
    Qh = np.zeros((B, Hq, n, d), dtype=np.float32)
    for (b, h) in sample:
        Qh[b, h * G:(h + 1) * G] = sdev.host_f32(Qd[b, h * G:(h + 1) * G])
    orc = _oracle_heads(Qh, Kh, cls_h, spec, sample, Ts[0])
    ds = sdev.make_decode_stream_device(spec, layer, steps, "cuda")
    dq_h = {(b, h): sdev.host_f32(ds.q[:, b, h * G:(h + 1) * G]) for (b, h) in decode_sample}
    dk_h = sdev.host_f32(ds.k)
    dv_h = sdev.host_f32(ds.v)
    ncls_h = ds.new_class_host
    max_kept = int(max(np.count_nonzero(ncls_h[:, b]) for b in range(B)))
    k_f, w_l = ref.budgets(n, spec.r_l, spec.r_f)
    report = {"flagged": 0, "checked": 0, "policies": {}, "dec_err": 0.0}
    tol = DEC_TOL[spec.dtype]
    for T in Ts:
        prof = fg.profile(Qd, Kd, cls_d, spec.r_l, spec.r_f, T, want_lse=True, want_band=True)
        torch.cuda.synchronize()
        pol_g = prof.policy.cpu().numpy()
        rec_g = prof.recovery.cpu().numpy().astype(np.float64)
        cum_g = prof.cum.cpu().numpy().astype(np.float64)
        F_g = prof.frequent()
        # properties of every head
        assert np.allclose(cum_g.sum(axis=-1), G * n, rtol=1e-4), "column sums must total G*n"
        assert np.all(np.diff(rec_g, axis=-1) >= -1e-6) and np.all(rec_g[..., 4] == 1.0)
        assert np.all(F_g.sum(axis=-1) == min(k_f, n))
        for b in range(B):
            for h in range(Hkv):
                if not np.any(np.abs(rec_g[b, h, :4] - T) < 1e-6):
                    own = next(k for k in range(5) if rec_g[b, h, k] >= T or k == 4)
                    assert int(pol_g[b, h]) == own, (b, h)
        # sampled heads against the oracle
        lse_g = prof.lse.cpu().numpy().astype(np.float64)
        band_g = prof.band.cpu().numpy().astype(np.float64)
        for (b, h), pr in orc.items():
            R = pr.R
            policy = ref.select_policy(R, T)
            near = ref.near_t_flag(R, T)
            assert np.max(np.abs(lse_g[b, h * G:(h + 1) * G] - pr.lse)) <= 2e-4 + 2e-6 * np.max(np.abs(pr.lse))
            assert np.allclose(cum_g[b, h], pr.cum, rtol=2e-4, atol=1e-6 * G), (b, h)
            assert np.allclose(band_g[b, h], pr.band, rtol=2e-4, atol=1e-6 * G), (b, h)
            assert np.max(np.abs(rec_g[b, h] - R)) <= REC_TOL, (b, h, rec_g[b, h], R)
            if pr.topk_tie:
                assert eps_topk_ok(pr.cum, F_g[b, h], pr.k_f, TIE_TAU), (b, h)
            else:
                assert np.array_equal(F_g[b, h], pr.F), (b, h)
            if near or pr.topk_tie:
                report["flagged"] += 1
                assert int(pol_g[b, h]) in allowed_policies(R, T, policy), (b, h)
            else:
                assert int(pol_g[b, h]) == policy, (b, h, rec_g[b, h], R)
            report["checked"] += 1
        report["policies"][T] = np.bincount(pol_g.reshape(-1), minlength=5).tolist()
        # compaction: the kept list of every head under the GPU's decisions, bytes of the sampled heads
        cache = fg.compact(Kd, Vd, cls_d, prof, Hq, max_new_tokens=steps, max_new_kept=max_kept)
        kept_g = cache.kept_positions()
        for b in range(B):
            for h in range(Hkv):
                want = ref.kept_positions(cls_h[b], F_g[b, h], w_l, int(pol_g[b, h]))
                assert np.array_equal(kept_g[b * Hkv + h], want), (b, h)
        for (b, h) in sample:
            pos, kc, vc = cache.rows(b * Hkv + h)
            sel = torch.from_numpy(pos >= 0).cuda()
            idx = torch.from_numpy(pos[pos >= 0]).cuda().long()
            assert torch.equal(kc[sel], Kd[b, h][idx]) and torch.equal(vc[sel], Vd[b, h][idx])
        # decode: every step on the device, outputs of the decode-sampled heads kept on the host
        sel_q = torch.tensor([b * Hq + h * G + g for (b, h) in decode_sample for g in range(G)],
                             dtype=torch.long, device="cuda")
        got = np.zeros((len(out_steps), len(decode_sample), G, d), dtype=np.float32)
        pos_of = {t: i for i, t in enumerate(out_steps)}
        for t in range(steps):
            o = cache.decode_step(ds.q[t], ds.k[t], ds.v[t], ds.new_class[t])
            if t in pos_of:
                got[pos_of[t]] = o.reshape(B * Hq, d)[sel_q].reshape(len(decode_sample), G, d).cpu().numpy()
        torch.cuda.synchronize()
        assert cache.error_bits() == 0
        final = cache.kept_positions()
        zq = np.zeros((steps, G, d))

        def final_cache(bh):
            b, h = bh
            _, c_ref = ref.decode_masked(Kh[b, h], Vh[b, h], cls_h[b], F_g[b, h], w_l, int(pol_g[b, h]), zq,
                                         dk_h[:, b, h], dv_h[:, b, h], ncls_h[:, b], steps_subset=[steps - 1])
            return bh, c_ref[-1]

        def outputs(i):
            b, h = decode_sample[i]
            o_ref, _ = ref.decode_masked(Kh[b, h], Vh[b, h], cls_h[b], F_g[b, h], w_l, int(pol_g[b, h]),
                                         dq_h[(b, h)], dk_h[:, b, h], dv_h[:, b, h], ncls_h[:, b],
                                         steps_subset=out_steps)
            scale = np.maximum(np.max(np.abs(o_ref), axis=-1), 1e-30)
            return i, np.max(np.abs(got[:, i] - o_ref), axis=-1) / scale

        worst = 0.0
        with _oracle_pool() as ex:
            for (b, h), want in ex.map(final_cache, [(b, h) for b in range(B) for h in range(Hkv)]):
                assert np.array_equal(final[b * Hkv + h], want), (b, h, "final cache")
            for i, err in ex.map(outputs, range(len(decode_sample))):
                worst = max(worst, float(err.max()))
                assert err.max() <= tol, (decode_sample[i], int(pol_g[decode_sample[i]]), float(err.max()),
                                          out_steps[int(np.argmax(err.max(axis=-1)))])
        report["dec_err"] = max(report["dec_err"], worst)
        log(f"[fullsize] T={T}: policies {report['policies'][T]}, sampled heads ok, kept lists of "
            f"{B * Hkv} heads ok, decode err {worst:.2e} over {len(decode_sample)} heads x {len(out_steps)} steps, "
            f"kept fraction {sum(len(k) for k in kept_g) / (B * Hkv * n):.3f}")
        del cache, prof
    log(f"[fullsize] ok: checked={report['checked']} flagged={report['flagged']}")
    return report
