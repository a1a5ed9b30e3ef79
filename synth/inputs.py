"""Seeded generator of Llama-shaped attention inputs with planted head types.

The FastGen pages (hyper.ai summary of "Model Tells You What to Discard",
Method section) describe four kinds of attention heads in trained Llama models:
heads that attend to special tokens, to punctuation, to a local window, and
broad heads.  No trained weights exist here, so this module plants those
structures into random post-RoPE Q/K/V:

* values: Q, K, V ~ N(0, 1) in fp32, rotary embedding (rotate-half pairing,
  base 1e4) at each token position, then the plants, then one
  round-to-nearest-even cast to bf16 (the tiny configuration stays fp32);
* special head: a direction u (N(0, I) rescaled to norm sqrt(d)) is added to
  every query and 6u to the keys of special tokens;
* punct head: the same, on punctuation tokens;
* heavy head: the same, on floor(n/20) random normal tokens;
* local head: q_i = rope(c + 0.3 xi_i), k_i = rope(c + 0.3 eta_i) with a shared
  c ~ N(0, 4 I);
* unplanted head: plain N(0, 1) + RoPE.

Token classes are u8 (0 normal, 1 special, 2 punct); position 0 is always
special (BOS), and exactly round(rate * n) further positions are drawn without
replacement for each other class.

Every array is a pure function of (configuration, layer, batch entry, tensor
kind) through ``numpy.random.SeedSequence``, so a sub-batch is exactly the
corresponding slice of the full batch.  Nothing here computes attention.
"""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

TOKEN_NORMAL = 0
TOKEN_SPECIAL = 1
TOKEN_PUNCT = 2

# tensor-kind tags folded into the seed
_K_Q, _K_K, _K_V, _K_CLS, _K_U, _K_C, _K_HEAVY, _K_MIX = 1, 2, 3, 4, 5, 6, 7, 8
_K_DQ, _K_DK, _K_DV, _K_DCLS, _K_PERM = 11, 12, 13, 14, 15

ROPE_BASE = 1.0e4


@dataclass(frozen=True)
class ConfigSpec:
    cfg_id: int
    name: str
    layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    head_dim: int
    dtype: str                      # "f32" or "bf16"
    T: Tuple[float, ...]
    r_l: float
    r_f: float
    decode_steps: int
    special_frac: float             # share of special tokens (position 0 included)
    punct_frac: float
    rope_heads: str = "all"         # "all" or "local_only"
    mix: str = "fixed"              # how head types are assigned
    fixed_types: Tuple[str, ...] = field(default_factory=tuple)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


CONFIGS: Dict[int, ConfigSpec] = {
    0: ConfigSpec(0, "tiny-planted", 1, 1, 4, 4, 256, 64, "f32", (0.95,), 0.3, 0.3, 32,
                  special_frac=0.0, punct_frac=0.08, rope_heads="local_only", mix="fixed",
                  fixed_types=("special", "punct", "local", "none")),
    1: ConfigSpec(1, "llama1-7b-layer", 1, 1, 32, 32, 2048, 128, "bf16", (0.95,), 0.3, 0.3, 256,
                  special_frac=0.01, punct_frac=0.06, mix="perm10"),
    2: ConfigSpec(2, "llama1-7b-stack", 32, 8, 32, 32, 4096, 128, "bf16", (0.90, 0.95, 0.99), 0.3, 0.3, 512,
                  special_frac=0.01, punct_frac=0.06, mix="depth"),
    3: ConfigSpec(3, "llama1-65b-stack", 80, 16, 64, 64, 2048, 128, "bf16", (0.95,), 0.3, 0.3, 1024,
                  special_frac=0.01, punct_frac=0.06, mix="depth"),
    4: ConfigSpec(4, "long-gqa-32k", 1, 1, 32, 8, 32768, 128, "bf16", (0.95,), 0.05, 0.1, 1024,
                  special_frac=0.01, punct_frac=0.05, mix="fixed",
                  fixed_types=("special", "punct", "heavy", "local", "none", "none", "none", "none")),
}

# Seed of configuration 0 is fixed so that the first punctuation token sits early
# (position <= 12); see ``canonical_seed``.
_CANONICAL_SEED = {0: 2, 1: 0, 2: 0, 3: 0, 4: 0}


def _parallel(fn, jobs) -> None:
    """Run independent fill jobs on a thread pool (each job owns its RNG stream and output slice)."""
    workers = min(16, os.cpu_count() or 1, max(1, len(jobs)))
    if workers <= 1:
        for j in jobs:
            fn(j)
        return
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for _ in ex.map(fn, jobs):
            pass


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding them."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (b + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of fp32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    if np.any(b & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-representable; call round_to_bf16 first")
    return (b >> np.uint32(16)).astype(np.uint16)


@functools.lru_cache(maxsize=16)
def _rope_tables_cached(first: int, count: int, d: int) -> Tuple[np.ndarray, np.ndarray]:
    half = d // 2
    inv = ROPE_BASE ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = (first + np.arange(count, dtype=np.float64))[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def _rope_tables(positions: np.ndarray, d: int) -> Tuple[np.ndarray, np.ndarray]:
    positions = np.asarray(positions)
    if len(positions) and np.array_equal(positions, positions[0] + np.arange(len(positions))):
        return _rope_tables_cached(int(positions[0]), len(positions), d)
    half = d // 2
    inv = ROPE_BASE ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = positions.astype(np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def _rope(x: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Rotate-half rotary embedding of x[..., n, d] at the given token positions (fp64 math)."""
    d = x.shape[-1]
    half = d // 2
    cos, sin = _rope_tables(positions, d)
    x = x.astype(np.float64)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def canonical_seed(cfg_id: int) -> int:
    return _CANONICAL_SEED[cfg_id]


def token_classes(spec: ConfigSpec, b: int, seed: Optional[int] = None) -> np.ndarray:
    """u8 classes of one prompt (batch entry b); identical across layers."""
    seed = canonical_seed(spec.cfg_id) if seed is None else seed
    n = spec.seq_len
    rng = _rng(seed, spec.cfg_id, b, _K_CLS)
    cls = np.zeros(n, dtype=np.uint8)
    cls[0] = TOKEN_SPECIAL
    n_special = max(1, int(round(spec.special_frac * n)))
    n_punct = int(round(spec.punct_frac * n))
    rest = rng.permutation(np.arange(1, n))
    cls[rest[: n_special - 1]] = TOKEN_SPECIAL
    cls[rest[n_special - 1: n_special - 1 + n_punct]] = TOKEN_PUNCT
    return cls


def head_types(spec: ConfigSpec, layer: int, seed: Optional[int] = None) -> List[str]:
    """Planted type of each KV head of one layer: special, punct, heavy, local or none."""
    seed = canonical_seed(spec.cfg_id) if seed is None else seed
    H = spec.n_kv_heads
    if spec.mix == "fixed":
        return list(spec.fixed_types)
    if spec.mix == "perm10":
        per = int(round(0.10 * H))
        types = ["special"] * per + ["punct"] * per + ["local"] * per
        types += ["none"] * (H - len(types))
        perm = _rng(seed, spec.cfg_id, layer, _K_PERM).permutation(H)
        return [types[i] for i in perm]
    if spec.mix == "depth":
        edge = layer < 4 or layer >= spec.layers - 4
        kinds = ["none", "local", "heavy", "punct", "special"]
        probs = [0.50, 0.25, 0.10, 0.10, 0.05] if edge else [0.10, 0.15, 0.10, 0.15, 0.50]
        draw = _rng(seed, spec.cfg_id, layer, _K_MIX).choice(len(kinds), size=H, p=probs)
        return [kinds[i] for i in draw]
    raise ValueError(spec.mix)


def _direction(seed: int, spec: ConfigSpec, layer: int, h: int) -> np.ndarray:
    u = _rng(seed, spec.cfg_id, layer, h, _K_U).standard_normal(spec.head_dim)
    return u * (np.sqrt(spec.head_dim) / np.linalg.norm(u))


def _local_center(seed: int, spec: ConfigSpec, layer: int, h: int) -> np.ndarray:
    return 2.0 * _rng(seed, spec.cfg_id, layer, h, _K_C).standard_normal(spec.head_dim)


@dataclass
class LayerInputs:
    spec: ConfigSpec
    layer: int
    batch_index: np.ndarray         # which batch entries these are
    Q: np.ndarray                   # [B, Hq, n, d] fp32 (bf16-representable for bf16 configs)
    K: np.ndarray                   # [B, Hkv, n, d]
    V: np.ndarray                   # [B, Hkv, n, d]
    token_class: np.ndarray         # [B, n] u8
    types: List[str]                # per KV head


def _uses_rope(spec: ConfigSpec, kind: str) -> bool:
    return spec.rope_heads == "all" or kind == "local"


def make_layer(spec: ConfigSpec, layer: int = 0, batch: Optional[Sequence[int]] = None,
               seed: Optional[int] = None, heads: Optional[Sequence[int]] = None) -> LayerInputs:
    """Prompt Q/K/V of one layer for the given batch entries (default: all).

    ``heads`` restricts the output to a subset of KV heads (and their query
    heads); the values equal the corresponding slice of the full layer.
    """
    seed = canonical_seed(spec.cfg_id) if seed is None else seed
    bidx = np.arange(spec.batch) if batch is None else np.asarray(batch, dtype=np.int64)
    kv_heads = np.arange(spec.n_kv_heads) if heads is None else np.asarray(heads, dtype=np.int64)
    G, n, d = spec.group, spec.seq_len, spec.head_dim
    types_all = head_types(spec, layer, seed)
    types = [types_all[h] for h in kv_heads]
    pos = np.arange(n)
    B, Hk = len(bidx), len(kv_heads)
    Q = np.empty((B, Hk * G, n, d), dtype=np.float32)
    K = np.empty((B, Hk, n, d), dtype=np.float32)
    V = np.empty((B, Hk, n, d), dtype=np.float32)
    cls = np.stack([token_classes(spec, int(b), seed) for b in bidx]) if B else np.zeros((0, n), np.uint8)
    def fill(job):
        bi, b, hi, h = job
        kind = types_all[h]
        kq = _rng(seed, spec.cfg_id, layer, int(b), int(h), _K_Q).standard_normal((G, n, d))
        kk = _rng(seed, spec.cfg_id, layer, int(b), int(h), _K_K).standard_normal((n, d))
        kv = _rng(seed, spec.cfg_id, layer, int(b), int(h), _K_V).standard_normal((n, d))
        if kind == "local":
            c = _local_center(seed, spec, layer, int(h))
            kq = c + 0.3 * kq
            kk = c + 0.3 * kk
        if _uses_rope(spec, kind):
            kq = _rope(kq, pos)
            kk = _rope(kk, pos)
        if kind in ("special", "punct", "heavy"):
            u = _direction(seed, spec, layer, int(h))
            kq = kq + u
            if kind == "special":
                sel = cls[bi] == TOKEN_SPECIAL
            elif kind == "punct":
                sel = cls[bi] == TOKEN_PUNCT
            else:
                normal = np.flatnonzero(cls[bi] == TOKEN_NORMAL)
                pick = _rng(seed, spec.cfg_id, layer, int(b), int(h), _K_HEAVY).choice(
                    normal, size=n // 20, replace=False)
                sel = np.zeros(n, dtype=bool)
                sel[pick] = True
            kk = kk.copy()
            kk[sel] += 6.0 * u
        rnd = round_to_bf16 if spec.dtype == "bf16" else (lambda x: x)
        Q[bi, hi * G:(hi + 1) * G] = rnd(kq.astype(np.float32))
        K[bi, hi] = rnd(kk.astype(np.float32))
        V[bi, hi] = rnd(kv.astype(np.float32))

    _parallel(fill, [(bi, b, hi, h) for bi, b in enumerate(bidx) for hi, h in enumerate(kv_heads)])
    return LayerInputs(spec, layer, bidx, Q, K, V, cls, types)


@dataclass
class DecodeStream:
    spec: ConfigSpec
    layer: int
    batch_index: np.ndarray
    q: np.ndarray                   # [steps, B, Hq, d]
    k: np.ndarray                   # [steps, B, Hkv, d]
    v: np.ndarray                   # [steps, B, Hkv, d]
    new_class: np.ndarray           # [steps, B] u8 (punct at the prompt's rate, never special)


def new_token_classes(spec: ConfigSpec, b: int, steps: int, seed: Optional[int] = None) -> np.ndarray:
    seed = canonical_seed(spec.cfg_id) if seed is None else seed
    draw = _rng(seed, spec.cfg_id, b, _K_DCLS).random(steps)
    return np.where(draw < spec.punct_frac, TOKEN_PUNCT, TOKEN_NORMAL).astype(np.uint8)


def make_decode_stream(spec: ConfigSpec, layer: int = 0, steps: Optional[int] = None,
                       batch: Optional[Sequence[int]] = None, seed: Optional[int] = None,
                       heads: Optional[Sequence[int]] = None) -> DecodeStream:
    """Per-step q, k_new, v_new of generated tokens at positions n, n+1, ..."""
    seed = canonical_seed(spec.cfg_id) if seed is None else seed
    steps = spec.decode_steps if steps is None else steps
    bidx = np.arange(spec.batch) if batch is None else np.asarray(batch, dtype=np.int64)
    kv_heads = np.arange(spec.n_kv_heads) if heads is None else np.asarray(heads, dtype=np.int64)
    G, n, d = spec.group, spec.seq_len, spec.head_dim
    types_all = head_types(spec, layer, seed)
    pos = n + np.arange(steps)
    B, Hk = len(bidx), len(kv_heads)
    q = np.empty((steps, B, Hk * G, d), dtype=np.float32)
    k = np.empty((steps, B, Hk, d), dtype=np.float32)
    v = np.empty((steps, B, Hk, d), dtype=np.float32)
    ncls = np.stack([new_token_classes(spec, int(b), steps, seed) for b in bidx], axis=1) \
        if B else np.zeros((steps, 0), np.uint8)
    def fill(job):
        bi, b, hi, h = job
        kind = types_all[h]
        dq = _rng(seed, spec.cfg_id, layer, int(b), int(h), _K_DQ).standard_normal((G, steps, d))
        dk = _rng(seed, spec.cfg_id, layer, int(b), int(h), _K_DK).standard_normal((steps, d))
        dv = _rng(seed, spec.cfg_id, layer, int(b), int(h), _K_DV).standard_normal((steps, d))
        if kind == "local":
            c = _local_center(seed, spec, layer, int(h))
            dq = c + 0.3 * dq
            dk = c + 0.3 * dk
        if _uses_rope(spec, kind):
            dq = _rope(dq, pos)
            dk = _rope(dk, pos)
        if kind in ("special", "punct", "heavy"):
            u = _direction(seed, spec, layer, int(h))
            dq = dq + u
            if kind == "punct":
                dk = dk.copy()
                dk[ncls[:, bi] == TOKEN_PUNCT] += 6.0 * u
        rnd = round_to_bf16 if spec.dtype == "bf16" else (lambda x: x)
        q[:, bi, hi * G:(hi + 1) * G] = rnd(np.transpose(dq, (1, 0, 2)).astype(np.float32))
        k[:, bi, hi] = rnd(dk.astype(np.float32))
        v[:, bi, hi] = rnd(dv.astype(np.float32))

    _parallel(fill, [(bi, b, hi, h) for bi, b in enumerate(bidx) for hi, h in enumerate(kv_heads)])
    return DecodeStream(spec, layer, bidx, q, k, v, ncls)


def custom_spec(base: ConfigSpec, **kw) -> ConfigSpec:
    """A copy of ``base`` with some fields replaced (for small test shapes)."""
    from dataclasses import replace
    return replace(base, **kw)
