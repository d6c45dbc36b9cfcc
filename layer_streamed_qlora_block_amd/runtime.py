"""Torch-facing convenience objects over the C ABI: device memory and streams.

``Store`` owns a pinned NF4 host store; ``Session`` owns a torch device
workspace and two torch streams (compute and copy, default priority) and
orders them against the caller's current stream around every call.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import (QLS_ABSMAX_DQ8, QLS_ABSMAX_F32, QLS_RESIDENT, QLS_STREAMED, RunCfg, model_cfg, qls_debug_set,
               qls_debug_capture_grads,
               pref_cfg, qls_adamw_step, qls_dpo_step, qls_pref_step, qls_layer_fwd_bwd, qls_layer_record_bytes_fmt, qls_logprobs, qls_lora_numel,
               qls_session_checkpoints, qls_session_create, qls_session_destroy, qls_session_reset_stats,
               qls_session_stats, qls_sft_step, qls_sft_step_adamw, qls_store_create_fmt, qls_store_create_tiered, qls_store_destroy, qls_store_layer_view,
               qls_store_set_layer_fp32, qls_store_set_layer_nf4, qls_workspace_bytes)


def _np_bf16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


class Store:
    """NF4 layer store.  absmax: "f32" (float32 per 64-block) or "dq8" (8-bit
    codes + one float32 scale per 256 blocks).  With disk_path, layers
    [0, ram_layers) are pinned host records and the rest spill to that file
    (the disk tier); otherwise every layer is pinned."""

    def __init__(self, cfg, max_pinned_bytes: int = 0, absmax: str = "f32", ram_layers=None, disk_path=None):
        if absmax not in ("f32", "dq8"):
            raise ValueError("absmax must be 'f32' or 'dq8'")
        self.cfg = cfg
        self.mc = model_cfg(cfg)
        self.absmax = absmax
        fmt = QLS_ABSMAX_DQ8 if absmax == "dq8" else QLS_ABSMAX_F32
        self.record_bytes = qls_layer_record_bytes_fmt(self.mc, fmt)
        self.lora_numel = qls_lora_numel(self.mc)
        if disk_path is not None:
            self.ram_layers = cfg.L if ram_layers is None else int(ram_layers)
            self.h = qls_store_create_tiered(self.mc, fmt, self.ram_layers, str(disk_path))
        else:
            self.ram_layers = cfg.L
            self.h = qls_store_create_fmt(self.mc, fmt, max_pinned_bytes)

    def set_layer_fp32(self, layer, weights, norm_attn, norm_mlp, n_threads: int = 0):
        ws = [np.ascontiguousarray(w, dtype=np.float32) for w in weights]
        na, nm = _np_bf16(norm_attn), _np_bf16(norm_mlp)
        qls_store_set_layer_fp32(self.h, layer, ws, na, nm, n_threads)

    def set_layer_nf4(self, layer, codes, absmax, norm_attn, norm_mlp):
        cs = [np.ascontiguousarray(c, dtype=np.uint8) for c in codes]
        am = [np.ascontiguousarray(a, dtype=np.float32) for a in absmax]
        qls_store_set_layer_nf4(self.h, layer, cs, am, _np_bf16(norm_attn), _np_bf16(norm_mlp))

    def view(self, layer):
        """The raw qls_layer_view of one record (host pointers into the store)."""
        return qls_store_layer_view(self.h, layer)

    def layer(self, layer) -> dict:
        """Copies of one record's NF4 codes and absmax data per module and its
        norms ("absmax" for f32 stores; "absmax_q8" and "absmax_scale" for dq8)."""
        v = qls_store_layer_view(self.h, layer)
        dq = v.absmax_format == QLS_ABSMAX_DQ8
        out = {"codes": [], "absmax": [], "absmax_q8": [], "absmax_scale": []}
        for m, (_, o, i) in enumerate(self.cfg.module_shapes()):
            n = o * i
            nb = n // 64
            out["codes"].append(np.ctypeslib.as_array(C.cast(v.codes[m], C.POINTER(C.c_uint8)), (n // 2,)).copy())
            if dq:
                out["absmax_q8"].append(np.ctypeslib.as_array(C.cast(v.absmax_q8[m], C.POINTER(C.c_uint8)), (nb,)).copy())
                out["absmax_scale"].append(np.ctypeslib.as_array(
                    C.cast(v.absmax_scale[m], C.POINTER(C.c_float)), (-(-nb // 256),)).copy())
            else:
                out["absmax"].append(np.ctypeslib.as_array(C.cast(v.absmax[m], C.POINTER(C.c_float)), (nb,)).copy())
        d = self.cfg.d
        out["norm_attn"] = np.ctypeslib.as_array(C.cast(v.norm_attn, C.POINTER(C.c_uint16)), (d,)).copy()
        out["norm_mlp"] = np.ctypeslib.as_array(C.cast(v.norm_mlp, C.POINTER(C.c_uint16)), (d,)).copy()
        return out

    def close(self):
        if self.h:
            qls_store_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Session:
    def __init__(self, store: Store, embed, lm_head, final_norm, max_tokens: int, max_seq: int,
                 mode: int = QLS_STREAMED, ce_chunk: int = 0, timing: bool = False, device="cuda"):
        if not torch.cuda.is_available():
            raise RuntimeError("a GPU is required: the streamed step runs only in the HIP kernels")
        self.store = store
        self.cfg = store.cfg
        self.run = RunCfg(mode, max_tokens, max_seq, ce_chunk, 1 if timing else 0)
        self.ws_bytes = qls_workspace_bytes(store.h, self.run)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.compute = torch.cuda.Stream(device=device)
        self.copy = torch.cuda.Stream(device=device)
        self.embed, self.lm_head, self.final_norm = embed, lm_head, final_norm
        torch.cuda.current_stream().synchronize()
        self.h = qls_session_create(store.h, self.run, self.ws, self.ws_bytes, self.compute, self.copy,
                                    embed, lm_head, final_norm)

    # Every call: compute waits for the caller's stream, caller waits for compute.
    def _enter(self):
        self.compute.wait_stream(torch.cuda.current_stream())

    def _exit(self):
        torch.cuda.current_stream().wait_stream(self.compute)

    def sft_step(self, ids, lora, grads, loss, host_loss=False):
        B, S = ids.shape
        self._enter()
        try:
            return qls_sft_step(self.h, ids, B, S, lora, grads, loss, want_host_loss=host_loss)
        finally:
            self._exit()

    def sft_step_adamw(self, ids, opt: "AdamW", grads, loss, host_loss=False):
        """SFT step with the AdamW update of opt.p (the LoRA vector) folded into
        the backward sweep (qls_sft_step_adamw); advances opt's step count."""
        B, S = ids.shape
        opt.t += 1
        self._enter()
        try:
            return qls_sft_step_adamw(self.h, ids, B, S, opt.p, grads, opt.m, opt.v, opt.t, opt.lr, opt.betas[0],
                                      opt.betas[1], opt.eps, opt.wd, loss, want_host_loss=host_loss)
        finally:
            self._exit()

    def logprobs(self, ids, prompt_len, lora, seq_logp, tok_logp=None):
        B, S = ids.shape
        self._enter()
        try:
            qls_logprobs(self.h, ids, B, S, prompt_len, lora, seq_logp, tok_logp)
        finally:
            self._exit()

    def dpo_step(self, chosen, rejected, prompt_len, beta, lora, grads, loss, aux=None, host_loss=False):
        S = chosen.shape[-1]
        self._enter()
        try:
            return qls_dpo_step(self.h, chosen, rejected, S, prompt_len, beta, lora, grads, loss, aux,
                                want_host_loss=host_loss)
        finally:
            self._exit()

    def pref_step(self, kind, chosen, rejected, prompt_len, lora, grads, loss, aux=None, host_loss=False,
                  **params):
        """Preference step of head kind ("dpo", "simpo", "orpo", "kto"); params:
        beta, gamma, lam, lam_d, lam_u (see qls_pref_step)."""
        S = chosen.shape[-1]
        cfg = pref_cfg(kind, **params)
        self._enter()
        try:
            return qls_pref_step(self.h, cfg, chosen, rejected, S, prompt_len, lora, grads, loss, aux,
                                 want_host_loss=host_loss)
        finally:
            self._exit()

    def layer_fwd_bwd(self, layer, x, gout, B, S, lora, out, gin, grads):
        self._enter()
        try:
            qls_layer_fwd_bwd(self.h, layer, x, gout, B, S, lora, out, gin, grads)
        finally:
            self._exit()

    def checkpoints(self, tokens):
        """bf16 view [(L+1), tokens, d] of the last step's layer-input checkpoints."""
        ptr, tm = qls_session_checkpoints(self.h)
        off = ptr - self.ws.data_ptr()
        L, d = self.cfg.L, self.cfg.d
        flat = self.ws[off:off + (L + 1) * tm * d * 2].view(torch.bfloat16).view(L + 1, tm, d)
        return flat[:, :tokens]

    def stats(self):
        return qls_session_stats(self.h)

    def reset_stats(self):
        qls_session_reset_stats(self.h)

    def debug(self, flags, delay_us=0):
        qls_debug_set(self.h, flags, delay_us)

    def capture_grads(self, buf):
        """Test hook: every backward sweep copies dL/dx_l for l = 0..L into buf,
        a float32 CUDA tensor of at least (L + 1) x tokens x hidden elements
        (None turns it off); the session keeps a reference while it is set."""
        if buf is not None and (buf.dtype != torch.float32 or not buf.is_cuda or not buf.is_contiguous()):
            raise ValueError("buf must be a contiguous float32 CUDA tensor")
        self._cap = buf
        qls_debug_capture_grads(self.h, buf)

    def close(self):
        if getattr(self, "h", None):
            qls_session_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


__all__ = ["Store", "Session", "QLS_STREAMED", "QLS_RESIDENT"]


class AdamW:
    """AdamW on the packed float32 LoRA vector (qls_adamw_step), moments in
    device memory, issued on torch's current stream (after the step's kernels,
    which the session orders before it)."""

    def __init__(self, params: torch.Tensor, lr: float = 2e-5, betas=(0.9, 0.999), eps: float = 1e-8,
                 weight_decay: float = 0.0):
        if params.dtype != torch.float32 or not params.is_cuda or not params.is_contiguous():
            raise ValueError("params must be a contiguous float32 CUDA tensor")
        self.p = params
        self.m = torch.zeros_like(params)
        self.v = torch.zeros_like(params)
        self.lr, self.betas, self.eps, self.wd = lr, betas, eps, weight_decay
        self.t = 0

    def step(self, grads: torch.Tensor):
        self.t += 1
        qls_adamw_step(self.p, grads, self.m, self.v, self.t, self.lr, self.betas[0], self.betas[1], self.eps,
                       self.wd, stream=torch.cuda.current_stream())
