"""Offline head-type maps and a hyper-parameter sensitivity sweep over the GPU path.

* ``build_head_map``: profile many prompts of one layer (batches of Q, K and
  token classes), add their per-head recovery with ``fg_head_map_accumulate``
  and type every KV head by the recovery averaged over the prompts
  (``fg_head_map_finish``).  This is the offline variant of the jisaku.com
  glossary entry "FastGen" (section Profiling phase): sample prompts are
  profiled once and the saved map is applied at inference, where FastGen
  proper profiles each prompt during its own encoding.
* ``sensitivity``: profile one batch of prompts under a grid of budget ratios
  r = r_l = r_f and recover ratios T and report, per setting, the policies
  chosen, the share of prompt keys kept and the attention the chosen policies
  retain (the kdj.com article, section Experimental Results and Efficacy,
  reports generation quality stable across hyper-parameter settings; retained
  attention is the quality proxy available without a trained model).

Every step runs in libfastgen's kernels; this module orchestrates calls and
summarises their outputs.  ``python -m adaptive_kv_cache_fg_amd.headmap``
runs both on the seeded synthetic layers of ``synth.inputs`` and prints one
JSON line.
"""
from __future__ import annotations

import argparse
import json
import sys
from typing import Iterable, List, Sequence, Tuple

import numpy as np
import torch

from . import fastgen as fg


def build_head_map(batches: Iterable[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]], n_kv_heads: int,
                   r_l: float, r_f: float, T: float) -> dict:
    """Head map of one layer from batches of prompts (Q [B,Hq,n,d], K [B,Hkv,n,d], token_class [B,n])."""
    hm = fg.HeadMap(n_kv_heads)
    kept_own = kept_map = keys = 0
    profs: List[Tuple[fg.Profile, torch.Tensor, torch.Tensor, int]] = []
    for Q, K, cls in batches:
        prof = fg.profile(Q, K, cls, r_l, r_f, T)
        hm.add(prof)
        profs.append((prof, K, cls, Q.shape[1]))
    mean, policy = hm.finish(T, r_l, r_f)
    # prompt keys kept with each prompt's own policies and with the map's
    for prof, K, cls, hq in profs:
        kept_own += int(fg.kept_counts(K, cls, prof, hq).sum().item())
        kept_map += int(fg.kept_counts(K, cls, fg.apply_head_map(prof, policy), hq).sum().item())
        keys += K.shape[0] * K.shape[1] * K.shape[2]
    count = hm.policy_count.cpu().numpy()
    pol = policy.cpu().numpy().astype(np.int64)
    return {
        "n_prompts": hm.n_prompts,
        "policy": pol.tolist(),
        "policy_histogram": np.bincount(pol, minlength=5).tolist(),
        "mean_recovery": mean.cpu().numpy().round(6).tolist(),
        "agreement": float(np.mean(count[np.arange(n_kv_heads), pol] / hm.n_prompts)),
        "kept_share_per_prompt_policies": kept_own / keys,
        "kept_share_map_policies": kept_map / keys,
    }


def sensitivity(Q: torch.Tensor, K: torch.Tensor, cls: torch.Tensor, rs: Sequence[float],
                Ts: Sequence[float]) -> List[dict]:
    """Policies, kept share and retained attention of one batch of prompts over a grid of (r, T)."""
    B, Hkv, n, _ = K.shape
    rows = []
    for r in rs:
        for T in Ts:
            prof = fg.profile(Q, K, cls, r, r, T)
            kept = fg.kept_counts(K, cls, prof, Q.shape[1])
            pol = prof.policy.cpu().numpy().reshape(-1).astype(np.int64)
            R = prof.recovery.cpu().numpy().reshape(-1, 5).astype(np.float64)
            retained = R[np.arange(len(pol)), pol]
            rows.append({"r": r, "T": T, "policy_histogram": np.bincount(pol, minlength=5).tolist(),
                         "kept_share": float(kept.sum().item()) / (B * Hkv * n),
                         "retained_mean": float(retained.mean()), "retained_min": float(retained.min())})
    return rows


def _upload(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def main(argv=None) -> int:
    from synth import inputs as syn
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--config", type=int, default=2, help="synthetic workload id")
    ap.add_argument("--layers", type=int, nargs="+", default=[0])
    ap.add_argument("--prompts", type=int, default=16, help="prompts per layer (rounded up to whole batches)")
    ap.add_argument("--r", type=float, nargs="+", default=[0.1, 0.2, 0.3, 0.4])
    ap.add_argument("--T", type=float, nargs="+", default=[0.90, 0.95, 0.99])
    args = ap.parse_args(argv)
    spec = syn.CONFIGS[args.config]
    base = syn.canonical_seed(spec.cfg_id)
    out = {"workload": spec.name, "batch_per_call": spec.batch, "r_l": spec.r_l, "r_f": spec.r_f,
           "T": spec.T[0], "layers": {}}
    first = None
    for layer in args.layers:
        calls = (args.prompts + spec.batch - 1) // spec.batch

        def batches():
            for i in range(calls):
                li = syn.make_layer(spec, layer, seed=base + 1000 * i)
                yield _upload(li.Q, spec.dtype), _upload(li.K, spec.dtype), torch.from_numpy(li.token_class).cuda()

        out["layers"][str(layer)] = build_head_map(batches(), spec.n_kv_heads, spec.r_l, spec.r_f, spec.T[0])
        if first is None:
            first = next(batches())
    Q, K, cls = first
    out["sensitivity_layer"] = args.layers[0]
    out["sensitivity"] = sensitivity(Q, K, cls, args.r, args.T)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
