"""Thin Python binding of libfastgen (ctypes).

Argument marshalling only: torch tensors provide device memory and the current
HIP stream; every step of profiling, compaction and decode runs in the HIP
kernels behind the C ABI declared in include/fastgen.h.  If the shared library
is missing this module raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from pathlib import Path
from typing import List, Optional

import numpy as np
import torch

_HERE = Path(__file__).resolve().parent
LIB_PATH = _HERE / "libfastgen.so"

FG_OK = 0
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small",
          4: "cache capacity exceeded", 5: "HIP error"}
DTYPE = {torch.bfloat16: 0, torch.float32: 1}
KERNEL_NAMES = ["profile_rowstats", "profile_colsums", "profile_select", "compact_plan", "compact_scan",
                "compact_gather", "compact_worklist", "decode_partials", "decode_merge", "attention", "decode_track",
                "profile_rowbins", "profile_rowbins_reduce"]


class FgShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class FgParams(ctypes.Structure):
    _fields_ = [("r_l", ctypes.c_double), ("r_f", ctypes.c_double), ("T", ctypes.c_double)]


class FgCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("row_offset", ctypes.c_void_p), ("len", ctypes.c_void_p), ("capacity", ctypes.c_void_p),
                ("ring", ctypes.c_void_p), ("policy", ctypes.c_void_p), ("work_offset", ctypes.c_void_p),
                ("work", ctypes.c_void_p), ("error_word", ctypes.c_void_p),
                ("total_rows", ctypes.c_int64), ("n_work", ctypes.c_int64), ("items_per_head", ctypes.c_int64),
                ("n_prompt", ctypes.c_int32), ("w_l", ctypes.c_int32), ("next_pos", ctypes.c_int32),
                ("chunk_rows", ctypes.c_int32), ("shape", FgShape)]


class FastGenError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfastgen.so (built in-tree by ``python -m adaptive_kv_cache_fg_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m adaptive_kv_cache_fg_amd.build`")
    L = ctypes.CDLL(str(LIB_PATH))
    P, S, I32, I64, D = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    sh, pa, ca = ctypes.POINTER(FgShape), ctypes.POINTER(FgParams), ctypes.POINTER(FgCache)
    L.fg_profile_workspace_size.argtypes, L.fg_profile_workspace_size.restype = [sh], S
    L.fg_profile.argtypes = [sh, pa, P, P, P, P, P, P, P, P, P, P, S, P]
    L.fg_profile.restype = ctypes.c_int
    L.fg_profile_attention.argtypes = [sh, pa, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
    L.fg_profile_attention.restype = ctypes.c_int
    L.fg_attention.argtypes, L.fg_attention.restype = [sh, P, P, P, P, P, P], ctypes.c_int
    L.fg_profile_row_bins.argtypes = [sh, pa, P, P, P, P, P, P, P]
    L.fg_profile_row_bins.restype = ctypes.c_int
    L.fg_profile_rows_workspace_size.argtypes, L.fg_profile_rows_workspace_size.restype = [sh], S
    L.fg_profile_rows.argtypes = [sh, pa, P, P, P, P, P, P, P, P, P, P, S, P]
    L.fg_profile_rows.restype = ctypes.c_int
    L.fg_decode_step_dynamic.argtypes = [ca, P, P, P, P, P, I32, P, P, P, S, P]
    L.fg_decode_step_dynamic.restype = ctypes.c_int
    L.fg_decode_track_init.argtypes, L.fg_decode_track_init.restype = [ca, P, P, P], ctypes.c_int
    L.fg_decode_track_workspace_size.argtypes, L.fg_decode_track_workspace_size.restype = [ca], S
    L.fg_decode_track.argtypes = [ca, P, P, I32, P, P, P, P, S, P]
    L.fg_decode_track.restype = ctypes.c_int
    L.fg_head_map_accumulate.argtypes = [I32, I32, P, P, P, P, P]
    L.fg_head_map_accumulate.restype = ctypes.c_int
    L.fg_head_map_finish.argtypes, L.fg_head_map_finish.restype = [I32, I64, pa, P, P, P, P], ctypes.c_int
    L.fg_compact_plan.argtypes = [sh, pa, P, P, P, I32, I32, P, P, P, P, P, P, P]
    L.fg_compact_plan.restype = ctypes.c_int
    L.fg_compact.argtypes = [sh, pa, P, P, P, P, P, ca, P]
    L.fg_compact.restype = ctypes.c_int
    L.fg_decode_workspace_size.argtypes, L.fg_decode_workspace_size.restype = [ca], S
    L.fg_decode_step.argtypes = [ca, P, P, P, P, P, P, S, P]
    L.fg_decode_step.restype = ctypes.c_int
    L.fg_decode_partials.argtypes, L.fg_decode_partials.restype = [ca, P, P, S, P], ctypes.c_int
    L.fg_cache_error.argtypes = [ca, ctypes.POINTER(ctypes.c_uint32), P]
    L.fg_cache_error.restype = ctypes.c_int
    L.fg_status_string.argtypes, L.fg_status_string.restype = [ctypes.c_int], ctypes.c_char_p
    L.fg_last_error.argtypes, L.fg_last_error.restype = [], ctypes.c_char_p
    L.fg_decode_chunk_rows.argtypes, L.fg_decode_chunk_rows.restype = [sh], I32
    L.fg_kernel_timing_enable.argtypes, L.fg_kernel_timing_enable.restype = [ctypes.c_int], None
    L.fg_kernel_timing_read.argtypes = [ctypes.POINTER(I32), ctypes.POINTER(ctypes.c_float), I32]
    L.fg_kernel_timing_read.restype = I32
    L.fg_kernel_name.argtypes, L.fg_kernel_name.restype = [I32], ctypes.c_char_p
    L.fg_decode_noalloc_max_bytes.argtypes, L.fg_decode_noalloc_max_bytes.restype = [], S
    L.fg_decode_step_noalloc.argtypes = [ca, P, P, P, P, P, P]
    L.fg_decode_step_noalloc.restype = ctypes.c_int
    L.fg_peak_mfma_bf16.argtypes, L.fg_peak_mfma_bf16.restype = [P, P, I32, I32, P], ctypes.c_int
    L.fg_peak_exp.argtypes, L.fg_peak_exp.restype = [P, I32, I32, P], ctypes.c_int
    L.fg_peak_mfma_softmax.argtypes, L.fg_peak_mfma_softmax.restype = [P, P, I32, I32, P], ctypes.c_int
    L.fg_peak_copy.argtypes, L.fg_peak_copy.restype = [P, P, S, I32, I32, P], ctypes.c_int
    L.fg_peak_read.argtypes, L.fg_peak_read.restype = [P, S, I32, I32, P, P], ctypes.c_int
    _ = D, I64
    _lib = L
    return L


def _check(status: int, where: str) -> None:
    if status != FG_OK:
        raise FastGenError(status, where, lib().fg_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def make_shape(Q: torch.Tensor, K: torch.Tensor) -> FgShape:
    B, Hq, n, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (B, Hkv, n, d):
        raise ValueError(f"K shape {tuple(K.shape)} does not match Q {tuple(Q.shape)}")
    if Q.dtype not in DTYPE or K.dtype != Q.dtype:
        raise ValueError("Q and K must both be bf16 or both fp32")
    return FgShape(B, Hq, Hkv, n, d, DTYPE[Q.dtype])


@dataclass
class Profile:
    policy: torch.Tensor        # [B, Hkv] uint8
    cum: torch.Tensor           # [B, Hkv, n] fp32
    recovery: torch.Tensor      # [B, Hkv, 5] fp32
    freq_mask: torch.Tensor     # [B, Hkv, ceil(n/32)] int32 (bit patterns of u32 words)
    lse: Optional[torch.Tensor]   # [B, Hq, n] fp32 natural log-sum-exp
    band: Optional[torch.Tensor]  # [B, Hkv, n] fp32
    r_l: float
    r_f: float
    T: float
    out: Optional[torch.Tensor] = None   # [B, Hq, n, d] attention output (profile with V only)
    row_min: Optional[torch.Tensor] = None   # [B, Hkv, 5] least kept share of a row (profile_rows only)
    bins: Optional[torch.Tensor] = None      # [B, Hq, n, 5] per-row level bins (profile_rows only)

    def frequent(self) -> np.ndarray:
        """Host bool array [B, Hkv, n] of the frequent set (synchronises)."""
        n = self.cum.shape[-1]
        words = self.freq_mask.cpu().numpy().view(np.uint32)
        bits = (words[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1
        return bits.reshape(*words.shape[:-1], -1)[..., :n].astype(bool)


def profile(Q: torch.Tensor, K: torch.Tensor, token_class: torch.Tensor, r_l: float, r_f: float, T: float,
            want_lse: bool = False, want_band: bool = False, V: Optional[torch.Tensor] = None,
            policy_out: Optional[torch.Tensor] = None) -> Profile:
    """fg_profile: per (b, KV head) cumulative scores, frequent set, recovery R_0..R_4 and policy.

    With V (bf16 only) this is fg_profile_attention: the prompt's attention
    output is computed in the same pass and returned as ``Profile.out``.
    ``policy_out`` (uint8, B*Hkv elements, contiguous) receives the policies in
    place of a new tensor: passing a cache's policy buffer (``cache.t["policy"]``)
    lets ``compact(..., reuse=cache)`` skip its copy of the policies; that cache
    is then stale until the compaction refills it.
    """
    _need(Q, "Q")
    _need(K, "K")
    _need(token_class, "token_class", torch.uint8)
    shape = make_shape(Q, K)
    B, Hq, n, _ = Q.shape
    Hkv = K.shape[1]
    dev = Q.device
    if policy_out is None:
        policy = torch.empty((B, Hkv), dtype=torch.uint8, device=dev)
    else:
        _need(policy_out, "policy_out", torch.uint8)
        if policy_out.numel() != B * Hkv or policy_out.device != dev:
            raise ValueError(f"policy_out must hold {B * Hkv} elements on {dev}")
        policy = policy_out.view(B, Hkv)
    cum = torch.empty((B, Hkv, n), dtype=torch.float32, device=dev)
    rec = torch.empty((B, Hkv, 5), dtype=torch.float32, device=dev)
    fmask = torch.empty((B, Hkv, (n + 31) // 32), dtype=torch.int32, device=dev)
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device=dev) if want_lse else None
    band = torch.empty((B, Hkv, n), dtype=torch.float32, device=dev) if want_band else None
    L = lib()
    ws_bytes = L.fg_profile_workspace_size(ctypes.byref(shape))
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    params = FgParams(r_l, r_f, T)
    if V is None:
        out = None
        _check(L.fg_profile(ctypes.byref(shape), ctypes.byref(params), _ptr(Q), _ptr(K), _ptr(token_class),
                            _ptr(policy), _ptr(cum), _ptr(rec), _ptr(fmask), _ptr(lse), _ptr(band),
                            _ptr(ws), ws_bytes, _stream()), "fg_profile")
    else:
        _need(V, "V", Q.dtype)
        if V.shape != K.shape:
            raise ValueError(f"V shape {tuple(V.shape)} does not match K {tuple(K.shape)}")
        out = torch.empty_like(Q)
        _check(L.fg_profile_attention(ctypes.byref(shape), ctypes.byref(params), _ptr(Q), _ptr(K), _ptr(V),
                                      _ptr(token_class), _ptr(out), _ptr(policy), _ptr(cum), _ptr(rec),
                                      _ptr(fmask), _ptr(lse), _ptr(band), _ptr(ws), ws_bytes, _stream()),
               "fg_profile_attention")
    return Profile(policy, cum, rec, fmask, lse, band, r_l, r_f, T, out)


def profile_rows(Q: torch.Tensor, K: torch.Tensor, token_class: torch.Tensor, r_l: float, r_f: float, T: float,
                 want_bins: bool = False, policy_out: Optional[torch.Tensor] = None) -> Profile:
    """fg_profile_rows: fg_profile with recovery from the per-row level bins, plus ``row_min``
    [B, Hkv, 5] (the least kept share of any row under each shortlist entry) and, with
    ``want_bins``, ``bins`` [B, Hq, n, 5]."""
    _need(Q, "Q")
    _need(K, "K")
    _need(token_class, "token_class", torch.uint8)
    shape = make_shape(Q, K)
    B, Hq, n, _ = Q.shape
    Hkv = K.shape[1]
    dev = Q.device
    if policy_out is None:
        policy = torch.empty((B, Hkv), dtype=torch.uint8, device=dev)
    else:
        _need(policy_out, "policy_out", torch.uint8)
        if policy_out.numel() != B * Hkv or policy_out.device != dev:
            raise ValueError(f"policy_out must hold {B * Hkv} elements on {dev}")
        policy = policy_out.view(B, Hkv)
    cum = torch.empty((B, Hkv, n), dtype=torch.float32, device=dev)
    rec = torch.empty((B, Hkv, 5), dtype=torch.float32, device=dev)
    fmask = torch.empty((B, Hkv, (n + 31) // 32), dtype=torch.int32, device=dev)
    row_min = torch.empty((B, Hkv, 5), dtype=torch.float32, device=dev)
    bins = torch.empty((B, Hq, n, 5), dtype=torch.float32, device=dev) if want_bins else None
    L = lib()
    ws_bytes = L.fg_profile_rows_workspace_size(ctypes.byref(shape))
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    params = FgParams(r_l, r_f, T)
    _check(L.fg_profile_rows(ctypes.byref(shape), ctypes.byref(params), _ptr(Q), _ptr(K), _ptr(token_class),
                             _ptr(policy), _ptr(cum), _ptr(rec), _ptr(fmask), _ptr(row_min), _ptr(bins), _ptr(ws),
                             ws_bytes, _stream()), "fg_profile_rows")
    prof = Profile(policy, cum, rec, fmask, None, None, r_l, r_f, T)
    prof.row_min = row_min
    prof.bins = bins
    return prof


def attention(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, want_lse: bool = False,
              out: Optional[torch.Tensor] = None):
    """fg_attention: causal softmax(Q K^T / sqrt(d)) V per query head (bf16) -> (O, lse or None)."""
    _need(Q, "Q")
    _need(K, "K")
    _need(V, "V", Q.dtype)
    shape = make_shape(Q, K)
    if V.shape != K.shape:
        raise ValueError(f"V shape {tuple(V.shape)} does not match K {tuple(K.shape)}")
    if out is None:
        out = torch.empty_like(Q)
    else:
        _need(out, "out", Q.dtype)
        if out.shape != Q.shape:
            raise ValueError("out must have Q's shape")
    B, Hq, n, _ = Q.shape
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device=Q.device) if want_lse else None
    _check(lib().fg_attention(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse), _stream()),
           "fg_attention")
    return out, lse


def row_bins(Q: torch.Tensor, K: torch.Tensor, token_class: torch.Tensor, prof: Profile) -> torch.Tensor:
    """fg_profile_row_bins: [B, Hq, n, 5] attention mass of each query row on the special, punct,
    frequent, local and remaining keys, from the frequent set and row log-sum-exps of ``prof``
    (a profile of the same Q, K, classes, made with want_lse=True)."""
    _need(Q, "Q")
    _need(K, "K")
    _need(token_class, "token_class", torch.uint8)
    if prof.lse is None:
        raise ValueError("row_bins needs the profile's row log-sum-exps: profile(..., want_lse=True)")
    shape = make_shape(Q, K)
    B, Hq, n, _ = Q.shape
    if tuple(prof.lse.shape) != (B, Hq, n) or prof.freq_mask.shape[:2] != K.shape[:2]:
        raise ValueError("the profile does not belong to these Q, K")
    bins = torch.empty((B, Hq, n, 5), dtype=torch.float32, device=Q.device)
    params = FgParams(prof.r_l, prof.r_f, prof.T)
    _check(lib().fg_profile_row_bins(ctypes.byref(shape), ctypes.byref(params), _ptr(Q), _ptr(K),
                                     _ptr(token_class), _ptr(prof.freq_mask), _ptr(prof.lse), _ptr(bins),
                                     _stream()), "fg_profile_row_bins")
    return bins


class HeadMap:
    """Multi-prompt head map of one layer (fg_head_map_accumulate / fg_head_map_finish)."""

    def __init__(self, n_kv_heads: int, device="cuda"):
        self.n_kv_heads = n_kv_heads
        self.rec_sum = torch.zeros((n_kv_heads, 5), dtype=torch.float64, device=device)
        self.policy_count = torch.zeros((n_kv_heads, 5), dtype=torch.int32, device=device)
        self.n_prompts = 0

    def add(self, prof: Profile) -> None:
        """Add the batch entries of one fg_profile call as prompts."""
        B, Hkv = prof.policy.shape
        if Hkv != self.n_kv_heads:
            raise ValueError(f"profile has {Hkv} KV heads, the map {self.n_kv_heads}")
        _check(lib().fg_head_map_accumulate(B, Hkv, _ptr(prof.recovery), _ptr(prof.policy), _ptr(self.rec_sum),
                                            _ptr(self.policy_count), _stream()), "fg_head_map_accumulate")
        self.n_prompts += B

    def finish(self, T: float, r_l: float = 0.0, r_f: float = 0.0):
        """(mean recovery [Hkv, 5] fp32, policy [Hkv] u8) over the prompts added so far."""
        mean = torch.empty((self.n_kv_heads, 5), dtype=torch.float32, device=self.rec_sum.device)
        policy = torch.empty((self.n_kv_heads,), dtype=torch.uint8, device=self.rec_sum.device)
        params = FgParams(r_l, r_f, T)
        _check(lib().fg_head_map_finish(self.n_kv_heads, self.n_prompts, ctypes.byref(params), _ptr(self.rec_sum),
                                        _ptr(mean), _ptr(policy), _stream()), "fg_head_map_finish")
        return mean, policy


def apply_head_map(prof: Profile, policy: torch.Tensor) -> Profile:
    """The profile with its policies replaced by a head map's (repeated over the batch), for fg_compact."""
    from dataclasses import replace
    B, Hkv = prof.policy.shape
    return replace(prof, policy=policy.reshape(1, Hkv).expand(B, Hkv).contiguous())


class Cache:
    """Head-specific ragged KV cache of one layer (owns its device tensors)."""

    def __init__(self, shape: FgShape, tensors: dict, struct: FgCache, kept_count: torch.Tensor):
        self.shape = shape
        self.t = tensors
        self.c = struct
        self.kept_count = kept_count
        self._ws = None
        self._tws = None

    @property
    def next_pos(self) -> int:
        return self.c.next_pos

    def decode_step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                    new_class: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """fg_decode_step for the token at position next_pos; returns out [B, Hq, d] fp32."""
        s = self.shape
        dt = self.t["k"].dtype
        _need(q, "q", dt)
        _need(k_new, "k_new", dt)
        _need(v_new, "v_new", dt)
        if q.shape != (s.batch, s.n_q_heads, s.head_dim) or k_new.shape != (s.batch, s.n_kv_heads, s.head_dim) \
                or v_new.shape != k_new.shape:
            raise ValueError("decode input shapes do not match the cache")
        if new_class is not None:
            _need(new_class, "new_class", torch.uint8)
            if new_class.shape != (s.batch,):
                raise ValueError("new_class must be [B]")
        if out is None:
            out = torch.empty((s.batch, s.n_q_heads, s.head_dim), dtype=torch.float32, device=q.device)
        L = lib()
        self._workspace(q.device)
        _check(L.fg_decode_step(ctypes.byref(self.c), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(new_class),
                                _ptr(out), _ptr(self._ws), self._ws.numel(), _stream()), "fg_decode_step")
        return out

    def decode_step_noalloc(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                            new_class: Optional[torch.Tensor], out: torch.Tensor) -> torch.Tensor:
        """fg_decode_step_noalloc: the same step with the library's static decode scratch instead of a
        workspace; allocates nothing (``out`` [B, Hq, d] fp32 is required)."""
        s = self.shape
        dt = self.t["k"].dtype
        _need(q, "q", dt)
        _need(k_new, "k_new", dt)
        _need(v_new, "v_new", dt)
        _need(out, "out", torch.float32)
        if q.shape != (s.batch, s.n_q_heads, s.head_dim) or k_new.shape != (s.batch, s.n_kv_heads, s.head_dim) \
                or v_new.shape != k_new.shape or out.shape != q.shape:
            raise ValueError("decode input shapes do not match the cache")
        if new_class is not None:
            _need(new_class, "new_class", torch.uint8)
            if new_class.shape != (s.batch,):
                raise ValueError("new_class must be [B]")
        _check(lib().fg_decode_step_noalloc(ctypes.byref(self.c), _ptr(q), _ptr(k_new), _ptr(v_new),
                                            _ptr(new_class), _ptr(out), _stream()), "fg_decode_step_noalloc")
        return out

    def decode_step_dynamic(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                            new_class: Optional[torch.Tensor], token_class: torch.Tensor, row_score: torch.Tensor,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """fg_decode_step_dynamic: decode with the frequent set re-ranked by row_score (see track())."""
        s = self.shape
        dt = self.t["k"].dtype
        _need(q, "q", dt)
        _need(k_new, "k_new", dt)
        _need(v_new, "v_new", dt)
        _need(token_class, "token_class", torch.uint8)
        _need(row_score, "row_score", torch.float32)
        if q.shape != (s.batch, s.n_q_heads, s.head_dim) or k_new.shape != (s.batch, s.n_kv_heads, s.head_dim) \
                or v_new.shape != k_new.shape or token_class.dim() != 2 or token_class.shape[0] != s.batch:
            raise ValueError("decode input shapes do not match the cache")
        if new_class is not None:
            _need(new_class, "new_class", torch.uint8)
        if out is None:
            out = torch.empty((s.batch, s.n_q_heads, s.head_dim), dtype=torch.float32, device=q.device)
        self._workspace(q.device)
        _check(lib().fg_decode_step_dynamic(ctypes.byref(self.c), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(new_class),
                                            _ptr(token_class), token_class.shape[1], _ptr(row_score), _ptr(out),
                                            _ptr(self._ws), self._ws.numel(), _stream()), "fg_decode_step_dynamic")
        return out

    def decode_partials(self, q: torch.Tensor) -> None:
        """fg_decode_partials: only the split-K launch of the next step (cache and next_pos unchanged)."""
        s = self.shape
        _need(q, "q", self.t["k"].dtype)
        if q.shape != (s.batch, s.n_q_heads, s.head_dim):
            raise ValueError("decode input shapes do not match the cache")
        self._workspace(q.device)
        _check(lib().fg_decode_partials(ctypes.byref(self.c), _ptr(q), _ptr(self._ws), self._ws.numel(), _stream()),
               "fg_decode_partials")

    def track_init(self, prof: Profile) -> torch.Tensor:
        """fg_decode_track_init: per-row cumulative scores [total_rows] starting from the prompt's."""
        score = torch.empty(max(int(self.c.total_rows), 1), dtype=torch.float32, device=self.t["k"].device)
        _check(lib().fg_decode_track_init(ctypes.byref(self.c), _ptr(prof.cum), _ptr(score), _stream()),
               "fg_decode_track_init")
        return score

    def track(self, q: torch.Tensor, token_class: torch.Tensor, freq_mask: torch.Tensor, row_score: torch.Tensor,
              level_bins: Optional[torch.Tensor] = None) -> torch.Tensor:
        """fg_decode_track after a decode step with that step's q: level bins [B, Hkv, 5] of its attention;
        row_score updated in place.  token_class [B, n_total] u8 covers every position so far."""
        s = self.shape
        _need(q, "q", self.t["k"].dtype)
        _need(token_class, "token_class", torch.uint8)
        if q.shape != (s.batch, s.n_q_heads, s.head_dim) or token_class.dim() != 2 or token_class.shape[0] != s.batch:
            raise ValueError("track input shapes do not match the cache")
        if level_bins is None:
            level_bins = torch.empty((s.batch, s.n_kv_heads, 5), dtype=torch.float32, device=q.device)
        if self._tws is None:
            nb = lib().fg_decode_track_workspace_size(ctypes.byref(self.c))
            self._tws = torch.empty(max(nb, 256), dtype=torch.uint8, device=q.device)
        _check(lib().fg_decode_track(ctypes.byref(self.c), _ptr(q), _ptr(token_class), token_class.shape[1],
                                     _ptr(freq_mask), _ptr(row_score), _ptr(level_bins), _ptr(self._tws),
                                     self._tws.numel(), _stream()), "fg_decode_track")
        return level_bins

    def _workspace(self, device) -> None:
        if self._ws is None:
            nb = lib().fg_decode_workspace_size(ctypes.byref(self.c))
            self._ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=device)

    def kept_positions(self) -> List[np.ndarray]:
        """Sorted kept-index list of every (b, KV head), from the device cache (synchronises)."""
        ro = self.t["row_offset"].cpu().numpy()
        ln = self.t["len"].cpu().numpy()
        pos = self.t["pos"].cpu().numpy()
        out = []
        for h in range(len(ln)):
            p = pos[ro[h]: ro[h] + ln[h]]
            out.append(np.sort(p[p >= 0]).astype(np.int64))
        return out

    def rows(self, head: int):
        """(pos, k, v) of the rows in use of one head, device order (synchronises)."""
        ro = int(self.t["row_offset"][head].item())
        ln = int(self.t["len"][head].item())
        return (self.t["pos"][ro:ro + ln].cpu().numpy(), self.t["k"][ro:ro + ln], self.t["v"][ro:ro + ln])

    def error_bits(self) -> int:
        bits = ctypes.c_uint32(0)
        st = lib().fg_cache_error(ctypes.byref(self.c), ctypes.byref(bits), _stream())
        if st not in (FG_OK, 4):
            _check(st, "fg_cache_error")
        return int(bits.value)


def compact(K: torch.Tensor, V: torch.Tensor, token_class: torch.Tensor, prof: Profile, n_q_heads: int,
            max_new_tokens: int, max_new_kept: Optional[int] = None, reuse: Optional[Cache] = None,
            check: bool = True) -> Cache:
    """fg_compact_plan + one read of the totals + fg_compact: the ragged cache of one layer.

    With ``reuse``, that cache's buffers are refilled in place (same device addresses, so a
    captured decode graph stays valid).  ``check=True`` plans into scratch tensors, reads the
    totals and copies the plan into the cache only when it fits; a plan that does not fit raises
    ValueError and leaves the cache's plan and rows untouched (if the profile already wrote its
    policies into the cache's buffer, the cache is marked unusable: decoding it fails until a
    compaction refills it).  ``check=False`` (reuse only) plans straight into the cache and skips
    the read of the new totals, so nothing synchronises the host and the call can be captured in
    a graph; a plan that does not fit the buffers then shows up as bit 2 of ``error_bits()``.
    """
    _need(K, "K")
    _need(V, "V", K.dtype)
    B, Hkv, n, d = K.shape
    if V.shape != K.shape:
        raise ValueError("V must match K")
    shape = FgShape(B, n_q_heads, Hkv, n, d, DTYPE[K.dtype])
    params = FgParams(prof.r_l, prof.r_f, prof.T)
    max_new_kept = max_new_tokens if max_new_kept is None else max_new_kept
    H = B * Hkv
    dev = K.device
    i32 = dict(dtype=torch.int32, device=dev)
    i64 = dict(dtype=torch.int64, device=dev)
    if reuse is not None:
        if (reuse.shape.batch, reuse.shape.n_kv_heads, reuse.shape.seq_len, reuse.shape.head_dim,
                reuse.shape.n_q_heads) != (B, Hkv, n, d, n_q_heads) or reuse.t["k"].dtype != K.dtype:
            raise ValueError("reuse: cache shape does not match")
    if reuse is not None and not check:
        plan = {"kept_count": reuse.kept_count, "ring": reuse.t["ring"], "capacity": reuse.t["capacity"],
                "row_offset": reuse.t["row_offset"], "work_offset": reuse.t["work_offset"],
                "totals": reuse.t["totals"]}
    else:
        plan = {"kept_count": torch.empty(H, **i32), "ring": torch.empty(H, **i32),
                "capacity": torch.empty(H, **i32), "row_offset": torch.empty(H + 1, **i64),
                "work_offset": torch.empty(H + 1, **i64), "totals": torch.empty(3, **i64)}
    L = lib()
    _check(L.fg_compact_plan(ctypes.byref(shape), ctypes.byref(params), _ptr(token_class), _ptr(prof.policy),
                             _ptr(prof.freq_mask), int(max_new_tokens), int(max_new_kept),
                             _ptr(plan["kept_count"]), _ptr(plan["ring"]), _ptr(plan["capacity"]),
                             _ptr(plan["row_offset"]), _ptr(plan["work_offset"]), _ptr(plan["totals"]),
                             _stream()), "fg_compact_plan")
    same_policy = reuse is not None and prof.policy.data_ptr() == reuse.t["policy"].data_ptr()
    if reuse is not None and not check:
        if not same_policy:
            reuse.t["policy"].copy_(prof.policy.reshape(-1))
        _check(L.fg_compact(ctypes.byref(shape), ctypes.byref(params), _ptr(K), _ptr(V), _ptr(token_class),
                            _ptr(reuse.t["policy"]), _ptr(prof.freq_mask), ctypes.byref(reuse.c), _stream()),
               "fg_compact")
        return reuse
    total_rows, n_work, per_head = (int(x) for x in plan["totals"].cpu().tolist())   # the one host synchronisation
    if reuse is not None:
        c = reuse.c
        if total_rows > c.total_rows or n_work > c.n_work or per_head > c.items_per_head:
            if same_policy:
                c.next_pos = -1        # its policies are the new prompt's, its rows the old one's: unusable
            raise ValueError("reuse: the new plan does not fit the cache's buffers")
        reuse.kept_count.copy_(plan["kept_count"])
        for name in ("ring", "capacity", "row_offset", "work_offset", "totals"):
            reuse.t[name].copy_(plan[name])
        if not same_policy:
            reuse.t["policy"].copy_(prof.policy.reshape(-1))
        _check(L.fg_compact(ctypes.byref(shape), ctypes.byref(params), _ptr(K), _ptr(V), _ptr(token_class),
                            _ptr(reuse.t["policy"]), _ptr(prof.freq_mask), ctypes.byref(c), _stream()), "fg_compact")
        return reuse
    t = {
        "k": torch.empty((max(total_rows, 1), d), dtype=K.dtype, device=dev),
        "v": torch.empty((max(total_rows, 1), d), dtype=K.dtype, device=dev),
        "pos": torch.empty(max(total_rows, 1), **i32),
        "row_offset": plan["row_offset"], "len": torch.empty(H, **i32), "capacity": plan["capacity"],
        "ring": plan["ring"], "policy": prof.policy.reshape(-1).clone(), "work_offset": plan["work_offset"],
        "totals": plan["totals"], "work": torch.empty(max(4 * n_work, 4), **i32),
        "error_word": torch.empty(1, **i32),
    }
    c = FgCache()
    for name in ("k", "v", "pos", "row_offset", "len", "capacity", "ring", "policy", "work_offset", "work",
                 "error_word"):
        setattr(c, name, t[name].data_ptr())
    c.total_rows, c.n_work, c.items_per_head = total_rows, n_work, per_head
    _check(L.fg_compact(ctypes.byref(shape), ctypes.byref(params), _ptr(K), _ptr(V), _ptr(token_class),
                        _ptr(t["policy"]), _ptr(prof.freq_mask), ctypes.byref(c), _stream()), "fg_compact")
    return Cache(shape, t, c, plan["kept_count"])


def kept_counts(K: torch.Tensor, token_class: torch.Tensor, prof: Profile, n_q_heads: int) -> torch.Tensor:
    """Prompt keys each (b, KV head) keeps under the profile's policies (fg_compact_plan only) -> [B*Hkv] int32."""
    _need(K, "K")
    B, Hkv, n, d = K.shape
    shape = FgShape(B, n_q_heads, Hkv, n, d, DTYPE[K.dtype])
    params = FgParams(prof.r_l, prof.r_f, prof.T)
    H = B * Hkv
    i32 = dict(dtype=torch.int32, device=K.device)
    i64 = dict(dtype=torch.int64, device=K.device)
    kept, ring, cap = torch.empty(H, **i32), torch.empty(H, **i32), torch.empty(H, **i32)
    row_offset, work_offset, totals = torch.empty(H + 1, **i64), torch.empty(H + 1, **i64), torch.empty(3, **i64)
    _check(lib().fg_compact_plan(ctypes.byref(shape), ctypes.byref(params), _ptr(token_class), _ptr(prof.policy),
                                 _ptr(prof.freq_mask), 0, 0, _ptr(kept), _ptr(ring), _ptr(cap), _ptr(row_offset),
                                 _ptr(work_offset), _ptr(totals), _stream()), "fg_compact_plan")
    return kept


def timing_enable(on: bool = True) -> None:
    """Bracket every eager launch with HIP events on its stream (not usable inside graph capture)."""
    lib().fg_kernel_timing_enable(1 if on else 0)


def timing_read(max_records: int = 1 << 16):
    """[(kernel name, ms)] of the launches bracketed since the last read (synchronises)."""
    ids = (ctypes.c_int32 * max_records)()
    ms = (ctypes.c_float * max_records)()
    k = lib().fg_kernel_timing_read(ids, ms, max_records)
    return [(KERNEL_NAMES[ids[i]], float(ms[i])) for i in range(k)]


def peak_mfma_bf16(operands: torch.Tensor, out: torch.Tensor, iters: int, blocks: int) -> float:
    """fg_peak_mfma_bf16; returns the flops of the call (4 chains x 32768 flops x iters per wave)."""
    _need(operands, "operands", torch.bfloat16)
    _need(out, "out", torch.float32)
    if operands.numel() < 8192 or out.numel() < blocks * 256:
        raise ValueError("operands must hold 8192 bf16 values and out blocks * 256 floats")
    _check(lib().fg_peak_mfma_bf16(_ptr(operands), _ptr(out), int(iters), int(blocks), _stream()),
           "fg_peak_mfma_bf16")
    return float(blocks) * 4 * 4 * 32768 * iters


def peak_mfma_softmax(operands: torch.Tensor, out: torch.Tensor, iters: int, blocks: int) -> float:
    """fg_peak_mfma_softmax; returns the MFMA flops of the call (waves 0-3 of each workgroup: 4 chains x
    32768 flops x iters; waves 4-7 run the sweeps' softmax updates beside them)."""
    _need(operands, "operands", torch.bfloat16)
    _need(out, "out", torch.float32)
    if operands.numel() < 8192 or out.numel() < blocks * 512:
        raise ValueError("operands must hold 8192 bf16 values and out blocks * 512 floats")
    _check(lib().fg_peak_mfma_softmax(_ptr(operands), _ptr(out), int(iters), int(blocks), _stream()),
           "fg_peak_mfma_softmax")
    return float(blocks) * 4 * 4 * 32768 * iters


def peak_exp(out: torch.Tensor, iters: int, blocks: int) -> float:
    """fg_peak_exp; returns the exponentials of the call (8 chains x iters per thread)."""
    _need(out, "out", torch.float32)
    if out.numel() < blocks * 256:
        raise ValueError("out must hold blocks * 256 floats")
    _check(lib().fg_peak_exp(_ptr(out), int(iters), int(blocks), _stream()), "fg_peak_exp")
    return float(blocks) * 256 * 8 * iters


def peak_copy(src: torch.Tensor, dst: torch.Tensor, nontemporal: bool, blocks: int) -> int:
    """fg_peak_copy of src's bytes into dst; returns the bytes moved (read + written)."""
    _need(src, "src")
    _need(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    _check(lib().fg_peak_copy(_ptr(src), _ptr(dst), nbytes, 1 if nontemporal else 0, int(blocks), _stream()),
           "fg_peak_copy")
    return 2 * nbytes


def peak_read(src: torch.Tensor, out: torch.Tensor, nontemporal: bool, blocks: int) -> int:
    """fg_peak_read of src's bytes (out: int32, at least blocks * 256 elements); returns the bytes read."""
    _need(src, "src")
    _need(out, "out", torch.int32)
    if out.numel() < blocks * 256:
        raise ValueError("out must hold blocks * 256 words")
    nbytes = src.numel() * src.element_size()
    _check(lib().fg_peak_read(_ptr(src), nbytes, 1 if nontemporal else 0, int(blocks), _ptr(out), _stream()),
           "fg_peak_read")
    return nbytes
