"""Python binding of libtd, the MI355X block-diffusion denoising step (C ABI in include/td.h).

Argument marshalling only: every step of the path runs in the HIP kernels behind the C
ABI.  torch tensors provide device memory and the HIP stream.  Importing this package
raises if libtd.so has not been built (build with `python block_diffusion_lm_step_amd/build.py`
or `__graft_entry__.build()`); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int8, c_int32, c_int64, c_uint8, c_void_p
from typing import Dict, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtd.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python block_diffusion_lm_step_amd/build.py` first")

# torch first: its HIP runtime is then the one libtd binds to, the same instance that
# owns the tensors and streams handed over (loading libtd first brings in a second
# runtime, which finds no device).
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)

TD_OK, TD_EINVAL, TD_ENOMEM, TD_EDEVICE, TD_EUNSUPPORTED = range(5)
TD_F32, TD_BF16 = 0, 1
STATUS_NAMES = {0: "TD_OK", 1: "TD_EINVAL", 2: "TD_ENOMEM", 3: "TD_EDEVICE", 4: "TD_EUNSUPPORTED"}


class TdConfig(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("d_model", c_int32), ("n_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("d_ff", c_int32), ("vocab", c_int32), ("block_size", c_int32),
                ("max_batch", c_int32), ("max_prefix_tokens", c_int64), ("dtype", c_int32), ("rms_eps", c_float)]


class TdWeights(ctypes.Structure):
    _fields_ = [("tok_emb", c_void_p), ("pos_emb", c_void_p), ("attn_norm", POINTER(c_void_p)),
                ("wq", POINTER(c_void_p)), ("wk", POINTER(c_void_p)), ("wv", POINTER(c_void_p)),
                ("wo", POINTER(c_void_p)), ("mlp_norm", POINTER(c_void_p)), ("w1", POINTER(c_void_p)),
                ("w2", POINTER(c_void_p)), ("final_norm", c_void_p), ("lm_head", c_void_p)]


class TdMoeConfig(ctypes.Structure):
    _fields_ = [("n_experts", c_int32), ("top_k", c_int32), ("n_shared", c_int32), ("d_expert", c_int32)]


class TdMoeWeights(ctypes.Structure):
    _fields_ = [("router", POINTER(c_void_p)), ("w1", POINTER(c_void_p)), ("w2", POINTER(c_void_p)),
                ("shared_w1", POINTER(c_void_p)), ("shared_w2", POINTER(c_void_p))]


_CTX = c_void_p
try:
    lib.td_create.argtypes = [POINTER(TdConfig), POINTER(TdWeights), c_void_p, POINTER(_CTX)]
    lib.td_set_prefix.argtypes = [_CTX, c_int32, POINTER(c_int64), POINTER(c_void_p), POINTER(c_void_p)]
    lib.td_denoise_step.argtypes = [_CTX, c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.td_denoise_step_noalloc.argtypes = [_CTX, c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                                            c_void_p, c_void_p]
    lib.td_generate_block.argtypes = [_CTX, c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p]
    lib.td_set_commit_rule.argtypes = [_CTX, c_int32, c_int32]
    lib.td_set_issue_window.argtypes = [_CTX, c_int32]
    lib.td_bind_cache.argtypes = [_CTX, c_int32, POINTER(c_int64), POINTER(c_int64), POINTER(c_void_p),
                                  POINTER(c_void_p)]
    lib.td_set_context_tower.argtypes = [_CTX, POINTER(TdWeights)]
    lib.td_append_block.argtypes = [_CTX, c_void_p]
    lib.td_ar_step.argtypes = [_CTX, c_void_p]
    lib.td_set_moe.argtypes = [_CTX, POINTER(TdMoeConfig), POINTER(TdMoeWeights)]
    lib.td_moe_stats.argtypes = [_CTX, POINTER(c_int64), POINTER(c_int64)]
    lib.td_debug_attention.argtypes = [_CTX, c_int32, c_void_p, c_void_p]
    lib.td_sync.argtypes = [_CTX]
    lib.td_profile_begin.argtypes = [_CTX, c_int32]
    lib.td_profile_begin.restype = c_int
    lib.td_profile_end.argtypes = [_CTX, POINTER(c_float), POINTER(c_int32), c_int32]
    lib.td_profile_layer.argtypes = [_CTX, c_int32]
    lib.td_profile_layer.restype = c_int
    lib.td_profile_end.restype = c_int32
    lib.td_kernels_per_step.argtypes = [_CTX]
    lib.td_kernels_per_step.restype = c_int32
    lib.td_destroy.argtypes = [_CTX]
    lib.td_destroy.restype = None
    lib.td_last_error.argtypes = [_CTX]
    lib.td_last_error.restype = c_char_p
    lib.td_version.restype = c_char_p
    lib.td_measure_peaks.argtypes = [c_void_p, c_int64, c_void_p, POINTER(ctypes.c_double), POINTER(ctypes.c_double),
                                     POINTER(ctypes.c_double)]
    lib.td_measure_peaks.restype = c_int
    for _f in ("td_create", "td_set_prefix", "td_bind_cache", "td_denoise_step", "td_denoise_step_noalloc",
               "td_generate_block",
               "td_set_commit_rule", "td_set_issue_window", "td_set_context_tower", "td_append_block",
               "td_ar_step", "td_set_moe", "td_moe_stats", "td_debug_attention", "td_sync"):
        getattr(lib, _f).restype = c_int
except AttributeError as e:   # a library built from older sources
    raise ImportError(f"{LIB_PATH} is stale ({e}); rebuild with `python block_diffusion_lm_step_amd/build.py`") from e

# Every symbol the C header declares.
EXPORTED = ("td_create", "td_set_prefix", "td_bind_cache", "td_denoise_step", "td_denoise_step_noalloc",
            "td_generate_block",
            "td_set_commit_rule", "td_set_issue_window", "td_set_context_tower", "td_append_block", "td_ar_step",
            "td_set_moe", "td_moe_stats", "td_debug_attention", "td_sync",
            "td_profile_begin", "td_profile_layer", "td_profile_end", "td_kernels_per_step", "td_measure_peaks",
            "td_destroy",
            "td_last_error", "td_version")
(TD_PROF_OFF, TD_PROF_LMHEAD, TD_PROF_GEMM, TD_PROF_ATTENTION, TD_PROF_STEP, TD_PROF_MOE, TD_PROF_ATTN_MERGE,
 TD_PROF_COMMIT, TD_PROF_EMBED) = range(9)
PROJ_QKV, PROJ_OUT, PROJ_UP, PROJ_DOWN, PROJ_ROUTER = range(5)   # sub tags of TD_PROF_GEMM
TD_RULE_THRESHOLD, TD_RULE_LEFT_TO_RIGHT = range(2)


class TdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _ptr_array(ts: Optional[Sequence]):
    """Device pointers of a list of tensors as a C array; None (or empty) -> NULL."""
    if not ts:
        return None
    return (c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def measure_peaks(buf, stream=None) -> Dict[str, float]:
    """td_measure_peaks over the device tensor buf (scratch, overwritten): HBM read stream
    and copy in GB/s, bf16 matrix-core loop in TFLOP/s."""
    import torch

    st = stream if stream is not None else torch.cuda.current_stream()
    r, c, m = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    status = lib.td_measure_peaks(c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(), c_void_p(st.cuda_stream),
                                  ctypes.byref(r), ctypes.byref(c), ctypes.byref(m))
    if status != TD_OK:
        raise TdError(status, "td_measure_peaks failed")
    return dict(hbm_read_gbs=r.value, copy_gbs=c.value, mfma_bf16_tflops=m.value)


class Denoiser:
    """One libtd context: a denoiser tower bound to one device and one HIP stream.

    cfg keys: n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ff, vocab, block_size,
    max_batch, max_prefix_tokens, dtype ("f32"/"bf16"), rms_eps.
    weights: torch tensors on the GPU in the config's dtype (bf16 as torch.bfloat16),
    keys as in td_weights; per-layer entries are lists.  w1 and w2 may be None when the
    MLP is a mixture of experts (set_moe before the first step).
    """

    def __init__(self, cfg: Dict, weights: Dict, stream=None):
        import torch

        self._torch = torch
        self.cfg = dict(cfg)
        c = TdConfig(cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"],
                     cfg["d_ff"], cfg["vocab"], cfg["block_size"], cfg["max_batch"], cfg["max_prefix_tokens"],
                     TD_BF16 if cfg["dtype"] == "bf16" else TD_F32, cfg.get("rms_eps", 1e-6))
        self._keep = {k: _ptr_array(weights.get(k)) for k in
                      ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w1", "w2")}
        w = TdWeights(weights["tok_emb"].data_ptr(), weights["pos_emb"].data_ptr(), self._keep["attn_norm"],
                      self._keep["wq"], self._keep["wk"], self._keep["wv"], self._keep["wo"],
                      self._keep["mlp_norm"], self._keep["w1"], self._keep["w2"], weights["final_norm"].data_ptr(),
                      weights["lm_head"].data_ptr())
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        ctx = _CTX()
        st = lib.td_create(ctypes.byref(c), ctypes.byref(w), c_void_p(self.stream.cuda_stream), ctypes.byref(ctx))
        if st != TD_OK:
            raise TdError(st, lib.td_last_error(None).decode())
        self._ctx = ctx
        self._prefix_refs = None

    def _check(self, st: int):
        if st != TD_OK:
            raise TdError(st, lib.td_last_error(self._ctx).decode())

    @property
    def kernels_per_step(self) -> int:
        return lib.td_kernels_per_step(self._ctx)

    def set_prefix(self, offsets: Sequence[int], k_caches: Sequence, v_caches: Sequence) -> None:
        n = len(offsets) - 1
        off = (c_int64 * (n + 1))(*[int(v) for v in offsets])
        ka, va = _ptr_array(k_caches), _ptr_array(v_caches)
        self._check(lib.td_set_prefix(self._ctx, n, off, ka, va))
        self._prefix_refs = (list(k_caches), list(v_caches))   # borrowed by the ctx

    def bind_cache(self, lengths: Sequence[int], page_capacity: Sequence[int], k_caches: Sequence,
                   v_caches: Sequence) -> None:
        n = len(lengths)
        ln = (c_int64 * n)(*[int(v) for v in lengths])
        cp = (c_int64 * n)(*[int(v) for v in page_capacity])
        ka, va = _ptr_array(k_caches), _ptr_array(v_caches)
        self._check(lib.td_bind_cache(self._ctx, n, ln, cp, ka, va))
        self._prefix_refs = (list(k_caches), list(v_caches))   # borrowed by the ctx

    def set_context_tower(self, weights: Dict) -> None:
        """weights: tok_emb and the per-layer lists, as for the denoiser; final_norm and lm_head
        optional (AR decoding)."""
        keep = {k: _ptr_array(weights[k]) for k in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w1", "w2")}
        head = [weights[k].data_ptr() if weights.get(k) is not None else None for k in ("final_norm", "lm_head")]
        w = TdWeights(weights["tok_emb"].data_ptr(), None, keep["attn_norm"], keep["wq"], keep["wk"], keep["wv"],
                      keep["wo"], keep["mlp_norm"], keep["w1"], keep["w2"], head[0], head[1])
        self._check(lib.td_set_context_tower(self._ctx, ctypes.byref(w)))

    def set_moe(self, cfg: Dict, weights: Dict) -> None:
        """cfg: n_experts, top_k, n_shared, d_expert.  weights: per-layer lists router
        [E][d], w1 [E][d_expert][d], w2 [E][d][d_expert], shared_w1, shared_w2 (None when
        n_shared is 0); copied and packed by the library."""
        c = TdMoeConfig(cfg["n_experts"], cfg["top_k"], cfg["n_shared"], cfg["d_expert"])
        keep = {k: _ptr_array(weights.get(k)) for k in ("router", "w1", "w2", "shared_w1", "shared_w2")}
        w = TdMoeWeights(keep["router"], keep["w1"], keep["w2"], keep["shared_w1"], keep["shared_w2"])
        self._check(lib.td_set_moe(self._ctx, ctypes.byref(c), ctypes.byref(w)))

    def moe_stats(self):
        """(expert-layer launches, sum of their active experts) since the previous call."""
        n, a = c_int64(0), c_int64(0)
        self._check(lib.td_moe_stats(self._ctx, ctypes.byref(n), ctypes.byref(a)))
        return n.value, a.value

    def append_block(self, tokens) -> None:
        self._check(lib.td_append_block(self._ctx, _ptr(tokens)))

    def ar_step(self, tokens) -> None:
        self._check(lib.td_ar_step(self._ctx, _ptr(tokens)))

    def denoise_step(self, tokens, committed, inv_temp, gamma: float, newly=None, conf=None, argmax=None,
                     logits=None) -> None:
        self._check(lib.td_denoise_step(self._ctx, _ptr(tokens), _ptr(committed), _ptr(inv_temp), float(gamma),
                                        _ptr(newly), _ptr(conf), _ptr(argmax), _ptr(logits)))

    def denoise_step_noalloc(self, tokens, committed, inv_temp, gamma: float, newly=None, conf=None, argmax=None,
                             logits=None) -> None:
        """td_denoise_step_noalloc: the step with its partial results in the library's
        file-scope device array (no allocation)."""
        self._check(lib.td_denoise_step_noalloc(self._ctx, _ptr(tokens), _ptr(committed), _ptr(inv_temp),
                                                float(gamma), _ptr(newly), _ptr(conf), _ptr(argmax), _ptr(logits)))

    def generate_block(self, tokens, committed, inv_temp, gamma: float, steps=None, commit_step=None) -> None:
        self._check(lib.td_generate_block(self._ctx, _ptr(tokens), _ptr(committed), _ptr(inv_temp), float(gamma),
                                          _ptr(steps), _ptr(commit_step)))

    def set_commit_rule(self, rule: int, min_adopt: int = 1) -> None:
        self._check(lib.td_set_commit_rule(self._ctx, int(rule), int(min_adopt)))

    def set_issue_window(self, steps_ahead: int) -> None:
        self._check(lib.td_set_issue_window(self._ctx, int(steps_ahead)))

    def debug_attention(self, layer: int, qkv, o) -> None:
        self._check(lib.td_debug_attention(self._ctx, int(layer), _ptr(qkv), _ptr(o)))

    def profile_begin(self, *kinds: int) -> None:
        """Bracket every launch of the given kernel classes (TD_PROF_*) with HIP events."""
        mask = 0
        for k in kinds:
            mask |= 1 << int(k)
        self._check(lib.td_profile_begin(self._ctx, mask))

    def profile_layer(self, layer: int) -> None:
        """Bracket the per-layer classes on this layer only (-1: every layer)."""
        self._check(lib.td_profile_layer(self._ctx, int(layer)))

    def profile_end(self, max_launches: int = 65536, tags: bool = False):
        """Durations (ms) of the bracketed launches in launch order; with tags=True also
        their tags (class, sub, layer) as a list of triples."""
        buf = (c_float * max_launches)()
        tg = (c_int32 * max_launches)()
        n = lib.td_profile_end(self._ctx, buf, tg, max_launches)
        if n < 0:
            raise TdError(TD_EDEVICE, lib.td_last_error(self._ctx).decode())
        m = min(n, max_launches)
        ms = [buf[i] for i in range(m)]
        if not tags:
            return ms
        return ms, [(tg[i] & 0xFF, (tg[i] >> 8) & 0xFF, tg[i] >> 16) for i in range(m)]

    def sync(self) -> None:
        self._check(lib.td_sync(self._ctx))

    def close(self) -> None:
        if getattr(self, "_ctx", None):
            lib.td_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
