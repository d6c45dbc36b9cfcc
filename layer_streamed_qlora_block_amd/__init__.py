"""Layer-streamed QLoRA step for AMD Instinct MI355X (gfx950) -- Python binding.

A thin ctypes layer over ``libqls.so`` (the C ABI declared in ``include/qls.h``):
every function here marshals arguments and calls the library of the same
name; all computation runs in the HIP kernels.  PyTorch only supplies device
memory and streams.  Importing fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes as C
import os

# torch first: its HIP runtime must be the process's one.  Loading libqls.so
# before torch would bind the system HIP runtime, and torch's own copy would
# then find no GPU.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqls.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(hipcc --offload-arch=gfx950); there is no fallback path")
_lib = C.CDLL(LIB_PATH)

QLS_OK, QLS_EINVAL, QLS_ENOMEM, QLS_ENOPIN, QLS_EHIP, QLS_ESTATE, QLS_EUNSUPPORTED, QLS_EIO = 0, -1, -2, -3, -4, -5, -6, -7
QLS_TIER_PINNED, QLS_TIER_DISK = 0, 1
QLS_STREAMED, QLS_RESIDENT = 0, 1
QLS_ABSMAX_F32, QLS_ABSMAX_DQ8 = 0, 1
QLS_PREF_DPO, QLS_PREF_SIMPO, QLS_PREF_ORPO, QLS_PREF_KTO = 0, 1, 2, 3
PREF_KINDS = {"dpo": QLS_PREF_DPO, "simpo": QLS_PREF_SIMPO, "orpo": QLS_PREF_ORPO, "kto": QLS_PREF_KTO}
NMOD = 7
MODULES = ("q", "k", "v", "o", "gate", "up", "down")
DBG_POISON_ON_RELEASE, DBG_COPY_DELAY, DBG_COMPUTE_DELAY, DBG_NO_REUSE, DBG_STREAM_FENCE = 1, 2, 4, 8, 16
DBG_RECOMPUTE_ALL = 32


class QlsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"qls error {code}: {msg}")
        self.code = code


class ModelCfg(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("intermediate", C.c_int32),
                ("vocab", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_float),
                ("lora_r", C.c_int32), ("lora_alpha", C.c_float)]


class PrefCfg(C.Structure):
    _fields_ = [("kind", C.c_int32), ("beta", C.c_float), ("gamma", C.c_float), ("lambda_", C.c_float),
                ("lambda_d", C.c_float), ("lambda_u", C.c_float)]


class RunCfg(C.Structure):
    _fields_ = [("mode", C.c_int32), ("max_tokens", C.c_int32), ("max_seq", C.c_int32),
                ("ce_chunk", C.c_int32), ("timing", C.c_int32)]


class Resident(C.Structure):
    _fields_ = [("d_embed", C.c_void_p), ("d_lm_head", C.c_void_p), ("d_final_norm", C.c_void_p)]


class LayerView(C.Structure):
    _fields_ = [("codes", C.c_void_p * NMOD), ("absmax", C.c_void_p * NMOD), ("norm_attn", C.c_void_p),
                ("norm_mlp", C.c_void_p), ("record", C.c_void_p), ("record_bytes", C.c_int64),
                ("absmax_format", C.c_int32), ("absmax_q8", C.c_void_p * NMOD),
                ("absmax_scale", C.c_void_p * NMOD)]


class Stats(C.Structure):
    _fields_ = [("steps", C.c_int64), ("layer_loads", C.c_int64), ("h2d_bytes", C.c_int64),
                ("copy_ms", C.c_double), ("compute_ms", C.c_double), ("overlap_ms", C.c_double),
                ("step_ms", C.c_double), ("ws_bytes", C.c_int64),
                ("dq_fwd_ms", C.c_double), ("dq_fwd_gflop", C.c_double), ("dq_fwd_launches", C.c_int64),
                ("dq_dx_ms", C.c_double), ("dq_dx_gflop", C.c_double), ("dq_dx_launches", C.c_int64),
                ("dq_fwd_big_ms", C.c_double), ("dq_fwd_big_gflop", C.c_double), ("dq_fwd_big_launches", C.c_int64),
                ("dq_dx_big_ms", C.c_double), ("dq_dx_big_gflop", C.c_double), ("dq_dx_big_launches", C.c_int64),
                ("dq_fwd_reduce_ms", C.c_double), ("dq_dx_reduce_ms", C.c_double),
                ("disk_reads", C.c_int64), ("disk_bytes", C.c_int64), ("disk_read_ms", C.c_double),
                ("disk_wait_ms", C.c_double), ("exposed_copy_ms", C.c_double), ("peak_ws_bytes", C.c_int64),
                ("dq_fwd_big_reduce_ms", C.c_double), ("dq_dx_big_reduce_ms", C.c_double)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_P = C.c_void_p
_I = C.c_int
_I64 = C.c_int64
_F = C.c_float
_SIG = {
    "qls_abi_version": (_I, []),
    "qls_last_error": (C.c_char_p, []),
    "qls_nf4_codebook": (_I, [_P]),
    "qls_nf4_quantize": (_I, [_P, _I64, _P, _P, _I]),
    "qls_nf4_dequant_dev": (_I, [_P, _P, _I64, _P, _P]),
    "qls_nf4_double_quant": (_I, [_P, _I64, _P, _P]),
    "qls_nf4_absmax_expand_dev": (_I, [_P, _P, _I64, _P, _P]),
    "qls_adamw_step": (_I, [_P, _P, _P, _P, _I64, _I, C.c_double, C.c_double, C.c_double, C.c_double,
                            C.c_double, _P]),
    "qls_attention_ws_bytes": (_I64, [_I, _I, _I, _I]),
    "qls_attention_fwd": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "qls_attention_bwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "qls_attention_bwd_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "qls_linear_ws_bytes": (_I64, [_I, _I, _I, _I]),
    "qls_linear_fwd": (_I, [_P, _P, _I, _I, _P, _I, _P, _P, _I, _F, _P, _P, _P, _P]),
    "qls_linear_bwd": (_I, [_P, _P, _I, _I, _P, _P, _P, _I, _P, _P, _I, _F, _P, _P, _P, _P, _P]),
    "qls_layer_record_bytes": (_I64, [C.POINTER(ModelCfg)]),
    "qls_layer_record_bytes_fmt": (_I64, [C.POINTER(ModelCfg), _I]),
    "qls_lora_numel": (_I64, [C.POINTER(ModelCfg)]),
    "qls_store_create": (_I, [C.POINTER(ModelCfg), C.c_uint64, C.POINTER(_P)]),
    "qls_store_create_fmt": (_I, [C.POINTER(ModelCfg), _I, C.c_uint64, C.POINTER(_P)]),
    "qls_store_create_tiered": (_I, [_P, _I, _I, C.c_char_p, _P]),
    "qls_store_layer_tier": (_I, [_P, _I]),
    "qls_store_set_layer_fp32": (_I, [_P, _I, _P * NMOD, _P, _P, _I]),
    "qls_store_set_layer_nf4": (_I, [_P, _I, _P * NMOD, _P * NMOD, _P, _P]),
    "qls_store_layer_view": (_I, [_P, _I, C.POINTER(LayerView)]),
    "qls_store_destroy": (None, [_P]),
    "qls_workspace_bytes": (_I, [_P, C.POINTER(RunCfg), C.POINTER(_I64)]),
    "qls_session_create": (_I, [_P, C.POINTER(RunCfg), _P, _I64, _P, _P, C.POINTER(Resident), C.POINTER(_P)]),
    "qls_session_destroy": (None, [_P]),
    "qls_sft_step": (_I, [_P, _P, _I, _I, _P, _P, _P, _P]),
    "qls_sft_step_adamw": (_I, [_P, _P, _I, _I, _P, _P, _P, _P, _I, C.c_double, C.c_double, C.c_double,
                                C.c_double, C.c_double, _P, _P]),
    "qls_logprobs": (_I, [_P, _P, _I, _I, _I, _P, _P, _P]),
    "qls_dpo_step": (_I, [_P, _P, _P, _I, _I, _F, _P, _P, _P, _P, _P]),
    "qls_pref_step": (_I, [_P, C.POINTER(PrefCfg), _P, _P, _I, _I, _P, _P, _P, _P, _P]),
    "qls_layer_fwd_bwd": (_I, [_P, _I, _P, _P, _I, _I, _P, _P, _P, _P]),
    "qls_session_checkpoints": (_I, [_P, C.POINTER(_P), C.POINTER(_I64)]),
    "qls_session_stats": (_I, [_P, C.POINTER(Stats)]),
    "qls_session_reset_stats": (_I, [_P]),
    "qls_debug_set": (_I, [_P, C.c_uint32, _I]),
    "qls_debug_capture_grads": (_I, [_P, _P, _I64]),
}
for _name, (_res, _args) in _SIG.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def exported_symbols():
    return list(_SIG)


def last_error() -> str:
    return _lib.qls_last_error().decode()


def _check(rc):
    if rc is not None and rc < 0:
        raise QlsError(rc, last_error())
    return rc


def _ptr(t):
    """Device/host pointer of a tensor or ndarray (None -> NULL)."""
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    return t.ctypes.data


def _stream(s):
    if s is None:
        return None
    return getattr(s, "cuda_stream", s)


def model_cfg(cfg) -> ModelCfg:
    """From a synth.ModelCfg-like object (L, d, H, KV, hd, I, V, eps, theta, r, alpha)."""
    return ModelCfg(cfg.L, cfg.d, cfg.H, cfg.KV, cfg.hd, cfg.I, cfg.V, cfg.eps, cfg.theta, cfg.r, cfg.alpha)


# ---------------------------------------------------------------- thin wrappers
def qls_abi_version() -> int:
    return _lib.qls_abi_version()


def qls_nf4_codebook():
    import numpy as np
    out = np.zeros(16, np.float32)
    _check(_lib.qls_nf4_codebook(out.ctypes.data))
    return out


def qls_nf4_quantize(w, n_threads: int = 0):
    import numpy as np
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    codes = np.empty(w.size // 2, np.uint8)
    absmax = np.empty(w.size // 64, np.float32)
    _check(_lib.qls_nf4_quantize(w.ctypes.data, w.size, codes.ctypes.data, absmax.ctypes.data, n_threads))
    return codes, absmax


def qls_nf4_dequant_dev(d_codes, d_absmax, n, d_out, stream=None):
    _check(_lib.qls_nf4_dequant_dev(_ptr(d_codes), _ptr(d_absmax), n, _ptr(d_out), _stream(stream)))


def qls_nf4_double_quant(absmax):
    import numpy as np
    a = np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1)
    q8 = np.empty(a.size, np.uint8)
    scales = np.empty(-(-a.size // 256), np.float32)
    _check(_lib.qls_nf4_double_quant(a.ctypes.data, a.size, q8.ctypes.data, scales.ctypes.data))
    return q8, scales


def qls_nf4_absmax_expand_dev(d_q8, d_scales, nblocks, d_out, stream=None):
    _check(_lib.qls_nf4_absmax_expand_dev(_ptr(d_q8), _ptr(d_scales), nblocks, _ptr(d_out), _stream(stream)))


def qls_adamw_step(params, grads, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                   stream=None):
    _check(_lib.qls_adamw_step(_ptr(params), _ptr(grads), _ptr(m), _ptr(v), params.numel(), step, lr, beta1,
                               beta2, eps, weight_decay, _stream(stream)))


def qls_attention_ws_bytes(B, S, H, hd) -> int:
    return _check(_lib.qls_attention_ws_bytes(B, S, H, hd))


def qls_attention_fwd(qkv, B, S, H, KV, hd, out, lse, stream=None):
    _check(_lib.qls_attention_fwd(_ptr(qkv), B, S, H, KV, hd, _ptr(out), _ptr(lse), _stream(stream)))


def qls_attention_bwd(qkv, out, dout, lse, B, S, H, KV, hd, dq, dk, dv, ws, stream=None):
    _check(_lib.qls_attention_bwd(_ptr(qkv), _ptr(out), _ptr(dout), _ptr(lse), B, S, H, KV, hd, _ptr(dq),
                                  _ptr(dk), _ptr(dv), _ptr(ws), _stream(stream)))


QLS_NOALLOC_SCRATCH_BYTES = 40 * 1024 * 1024


def qls_attention_bwd_noalloc(qkv, out, dout, lse, B, S, H, KV, hd, dq, dk, dv, stream=None):
    _check(_lib.qls_attention_bwd_noalloc(_ptr(qkv), _ptr(out), _ptr(dout), _ptr(lse), B, S, H, KV, hd, _ptr(dq),
                                          _ptr(dk), _ptr(dv), _stream(stream)))


def qls_linear_ws_bytes(T, N, K, r) -> int:
    return _check(_lib.qls_linear_ws_bytes(T, N, K, r))


def qls_linear_fwd(codes, absmax, N, K, x, T, A, B, r, alpha, y, u, ws, stream=None):
    _check(_lib.qls_linear_fwd(_ptr(codes), _ptr(absmax), N, K, _ptr(x), T, _ptr(A), _ptr(B), r, alpha,
                               _ptr(y), _ptr(u), _ptr(ws), _stream(stream)))


def qls_linear_bwd(codes, absmax, N, K, x, u, dy, T, A, B, r, alpha, dx, dA, dB, ws, stream=None):
    _check(_lib.qls_linear_bwd(_ptr(codes), _ptr(absmax), N, K, _ptr(x), _ptr(u), _ptr(dy), T, _ptr(A),
                               _ptr(B), r, alpha, _ptr(dx), _ptr(dA), _ptr(dB), _ptr(ws), _stream(stream)))


def qls_layer_record_bytes(mc: ModelCfg) -> int:
    return _check(_lib.qls_layer_record_bytes(C.byref(mc)))


def qls_layer_record_bytes_fmt(mc: ModelCfg, absmax_format: int) -> int:
    return _check(_lib.qls_layer_record_bytes_fmt(C.byref(mc), absmax_format))


def qls_lora_numel(mc: ModelCfg) -> int:
    return _check(_lib.qls_lora_numel(C.byref(mc)))


def qls_store_create(mc: ModelCfg, max_pinned_bytes: int = 0):
    h = _P()
    _check(_lib.qls_store_create(C.byref(mc), max_pinned_bytes, C.byref(h)))
    return h


def qls_store_create_tiered(mc: ModelCfg, absmax_format: int, ram_layers: int, path: str):
    h = _P()
    _check(_lib.qls_store_create_tiered(C.byref(mc), absmax_format, ram_layers, path.encode(), C.byref(h)))
    return h


def qls_store_layer_tier(store, layer: int) -> int:
    return _check(_lib.qls_store_layer_tier(store, layer))


def qls_store_create_fmt(mc: ModelCfg, absmax_format: int, max_pinned_bytes: int = 0):
    h = _P()
    _check(_lib.qls_store_create_fmt(C.byref(mc), absmax_format, max_pinned_bytes, C.byref(h)))
    return h


def qls_store_set_layer_fp32(store, layer, ws, norm_attn, norm_mlp, n_threads: int = 0):
    arr = (_P * NMOD)(*[_ptr(w) for w in ws])
    _check(_lib.qls_store_set_layer_fp32(store, layer, arr, _ptr(norm_attn), _ptr(norm_mlp), n_threads))


def qls_store_set_layer_nf4(store, layer, codes, absmax, norm_attn, norm_mlp):
    ca = (_P * NMOD)(*[_ptr(c) for c in codes])
    aa = (_P * NMOD)(*[_ptr(a) for a in absmax])
    _check(_lib.qls_store_set_layer_nf4(store, layer, ca, aa, _ptr(norm_attn), _ptr(norm_mlp)))


def qls_store_layer_view(store, layer) -> LayerView:
    v = LayerView()
    _check(_lib.qls_store_layer_view(store, layer, C.byref(v)))
    return v


def qls_store_destroy(store):
    _lib.qls_store_destroy(store)


def qls_workspace_bytes(store, run: RunCfg) -> int:
    out = _I64()
    _check(_lib.qls_workspace_bytes(store, C.byref(run), C.byref(out)))
    return out.value


def qls_session_create(store, run: RunCfg, ws, ws_bytes, compute_stream, copy_stream, embed, lm_head,
                       final_norm):
    res = Resident(_ptr(embed), _ptr(lm_head), _ptr(final_norm))
    h = _P()
    _check(_lib.qls_session_create(store, C.byref(run), _ptr(ws), ws_bytes, _stream(compute_stream),
                                   _stream(copy_stream), C.byref(res), C.byref(h)))
    return h


def qls_session_destroy(sess):
    _lib.qls_session_destroy(sess)


def qls_sft_step(sess, ids, B, S, lora, grads, loss, want_host_loss=False):
    hl = C.c_float(0.0)
    _check(_lib.qls_sft_step(sess, _ptr(ids), B, S, _ptr(lora), _ptr(grads), _ptr(loss),
                             C.byref(hl) if want_host_loss else None))
    return hl.value if want_host_loss else None


def qls_sft_step_adamw(sess, ids, B, S, lora, grads, m, v, step, lr, beta1, beta2, eps, weight_decay, loss,
                       want_host_loss=False):
    hl = C.c_float(0.0)
    _check(_lib.qls_sft_step_adamw(sess, _ptr(ids), B, S, _ptr(lora), _ptr(grads), _ptr(m), _ptr(v), step, lr,
                                   beta1, beta2, eps, weight_decay, _ptr(loss),
                                   C.byref(hl) if want_host_loss else None))
    return hl.value if want_host_loss else None


def qls_logprobs(sess, ids, B, S, prompt_len, lora, seq_logp, tok_logp=None):
    _check(_lib.qls_logprobs(sess, _ptr(ids), B, S, prompt_len, _ptr(lora), _ptr(seq_logp), _ptr(tok_logp)))


def qls_dpo_step(sess, chosen, rejected, S, prompt_len, beta, lora, grads, loss, aux=None,
                 want_host_loss=False):
    hl = C.c_float(0.0)
    _check(_lib.qls_dpo_step(sess, _ptr(chosen), _ptr(rejected), S, prompt_len, beta, _ptr(lora),
                             _ptr(grads), _ptr(loss), C.byref(hl) if want_host_loss else None, _ptr(aux)))
    return hl.value if want_host_loss else None


def qls_pref_step(sess, cfg: PrefCfg, chosen, rejected, S, prompt_len, lora, grads, loss, aux=None,
                  want_host_loss=False):
    hl = C.c_float(0.0)
    _check(_lib.qls_pref_step(sess, C.byref(cfg), _ptr(chosen), _ptr(rejected), S, prompt_len, _ptr(lora),
                              _ptr(grads), _ptr(loss), C.byref(hl) if want_host_loss else None, _ptr(aux)))
    return hl.value if want_host_loss else None


def pref_cfg(kind: str, beta: float = 0.0, gamma: float = 0.0, lam: float = 0.0, lam_d: float = 1.0,
             lam_u: float = 1.0) -> PrefCfg:
    if kind not in PREF_KINDS:
        raise ValueError(f"kind must be one of {sorted(PREF_KINDS)}")
    return PrefCfg(PREF_KINDS[kind], beta, gamma, lam, lam_d, lam_u)


def qls_layer_fwd_bwd(sess, layer, x, gout, B, S, lora, out, gin, grads):
    _check(_lib.qls_layer_fwd_bwd(sess, layer, _ptr(x), _ptr(gout), B, S, _ptr(lora), _ptr(out), _ptr(gin),
                                  _ptr(grads)))


def qls_session_checkpoints(sess):
    p = _P()
    n = _I64()
    _check(_lib.qls_session_checkpoints(sess, C.byref(p), C.byref(n)))
    return p.value, n.value


def qls_session_stats(sess) -> dict:
    s = Stats()
    _check(_lib.qls_session_stats(sess, C.byref(s)))
    return s.as_dict()


def qls_session_reset_stats(sess):
    _check(_lib.qls_session_reset_stats(sess))


def qls_debug_set(sess, flags, delay_us=0):
    _check(_lib.qls_debug_set(sess, flags, delay_us))


def qls_debug_capture_grads(sess, buf, n_floats=None):
    if buf is not None and n_floats is None:
        n_floats = buf.numel()
    _check(_lib.qls_debug_capture_grads(sess, _ptr(buf), 0 if buf is None else n_floats))


from .runtime import AdamW, Session, Store  # noqa: E402  (torch-facing convenience objects)
