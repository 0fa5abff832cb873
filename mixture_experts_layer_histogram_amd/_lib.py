"""ctypes binding of libmoe_hip.so (the C ABI declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the shared library.  Tensors are passed as device pointers (``data_ptr()``) on
the current HIP stream; ``None`` becomes NULL.  There is no fallback: if the
library is missing, :func:`lib` raises.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB

c_int32, c_int64, c_float, c_size_t, c_void_p = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                                 ctypes.c_size_t, ctypes.c_void_p)

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_INTERNAL = 0, -1, -2, -3, -4, -5
MOE_F32, MOE_BF16 = 0, 1
GATE_RULES = {"topk_softmax": 0, "softmax_renorm": 1, "switch_top1": 2}
ACTS = {"swiglu": 0, "gelu": 1}
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16}


class MoeConfig(ctypes.Structure):
    _fields_ = [("n_tokens", c_int64), ("d_model", c_int32), ("n_experts", c_int32), ("top_k", c_int32),
                ("d_ff", c_int32), ("d_ff_shared", c_int32), ("act", c_int32), ("ffn_bias", c_int32),
                ("gate_rule", c_int32), ("capacity_factor", c_float), ("dtype", c_int32),
                ("add_residual", c_int32), ("capacity_layout", c_int32), ("capacity_priority", c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("w_router", "logit_bias", "w1", "w3", "w2", "b1", "b2",
                                        "sh_w1", "sh_w3", "sh_w2")]


class MoeOutputs(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("out", "logits", "topk_idx", "gates", "counts", "offsets", "perm",
                                        "slot_pos", "drop_count", "probsum", "aux", "signs",
                                        "sel_bias_next")] + [("bias_gamma", c_float)]


class MoeSaved(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("logits", "topk_idx", "gates", "counts", "offsets", "perm", "slot_pos",
                                        "y_perm", "pre_act")]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("dx", "dw_router", "dlogit_bias", "dw1", "dw3", "dw2", "db1", "db2",
                                        "dsh_w1", "dsh_w3", "dsh_w2", "dgates")]


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {status}: {status_str(status)}")


_LIB = None
_P = c_void_p
_SIGS = {
    "moe_workspace_size": [ctypes.POINTER(MoeConfig), ctypes.POINTER(c_size_t)],
    "moe_expert_rows": [ctypes.POINTER(MoeConfig), ctypes.POINTER(c_int64), ctypes.POINTER(c_int32)],
    "moe_route": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P],
    "moe_permute": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P],
    "moe_permute_noalloc": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_expert_ffn": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P],
    "moe_expert_up": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, c_size_t, _P],
    "moe_expert_up_gather": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P],
    "moe_expert_up_save": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P],
    "moe_expert_down": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, c_size_t, _P],
    "moe_expert_down_combine": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t,
                                _P],
    "moe_quantize_fp8": [_P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P],
    "moe_probe_hbm_read": [_P, c_size_t, _P, _P],
    "moe_probe_mfma_bf16": [_P, ctypes.c_int64, _P, _P],
    "moe_probe_mfma_flop_per_iter": [ctypes.POINTER(c_int64)],
    "moe_expert_up_fp8": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P],
    "moe_expert_down_fp8": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, c_size_t, _P],
    "moe_shared_ffn": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, c_size_t, _P],
    "moe_combine": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P],
    "moe_bias_update": [ctypes.POINTER(MoeConfig), _P, c_float, _P, _P, _P],
    "moe_aux_loss": [ctypes.POINTER(MoeConfig), _P, _P, _P, _P],
    "moe_forward": [ctypes.POINTER(MoeConfig), ctypes.POINTER(MoeWeights), _P, _P, _P,
                    ctypes.POINTER(MoeOutputs), _P, c_size_t, _P],
    "moe_backward_workspace_size": [ctypes.POINTER(MoeConfig), ctypes.POINTER(c_size_t)],
    "moe_backward": [ctypes.POINTER(MoeConfig), ctypes.POINTER(MoeWeights), _P, _P, c_float,
                     ctypes.POINTER(MoeSaved), ctypes.POINTER(MoeGrads), _P, c_size_t, _P],
}


def lib() -> ctypes.CDLL:
    """Load libmoe_hip.so (built in-tree by build.py); raise if it is absent."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"HIP library {LIB} is not built; run "
                               "`python -m mixture_experts_layer_histogram_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = c_int32
        L.moe_status_str.argtypes = [c_int32]
        L.moe_status_str.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != MOE_OK:
        raise MoeError(name, st)


LAYOUTS = {"packed": 0, "padded": 1}
PRIORITIES = {"slot": 0, "choice": 1}


def make_config(n_tokens, d_model, n_experts, top_k, d_ff, d_ff_shared=0, act="swiglu", ffn_bias=False,
                gate_rule="topk_softmax", capacity_factor=0.0, dtype="bf16", add_residual=True,
                capacity_layout="packed", capacity_priority="slot") -> MoeConfig:
    return MoeConfig(int(n_tokens), int(d_model), int(n_experts), int(top_k), int(d_ff), int(d_ff_shared),
                     ACTS[act], int(bool(ffn_bias)), GATE_RULES[gate_rule], float(capacity_factor),
                     DTYPES[dtype], int(bool(add_residual)), LAYOUTS[capacity_layout],
                     PRIORITIES[capacity_priority])


def expert_rows(cfg: MoeConfig) -> int:
    """moe_expert_rows: rows of the expert-ordered buffers (perm, x_perm, h, y) for this config."""
    n = c_int64(0)
    _call("moe_expert_rows", ctypes.byref(cfg), ctypes.byref(n), None)
    return n.value


def capacity(cfg: MoeConfig) -> int:
    """moe_expert_rows' capacity C = floor(cf * N / E) (INT32_MAX when unlimited)."""
    n, c = c_int64(0), c_int32(0)
    _call("moe_expert_rows", ctypes.byref(cfg), ctypes.byref(n), ctypes.byref(c))
    return c.value


def workspace_size(cfg: MoeConfig) -> int:
    n = c_size_t(0)
    _call("moe_workspace_size", ctypes.byref(cfg), ctypes.byref(n))
    return n.value


def _ws(ws):
    return (None, 0) if ws is None else (ws.data_ptr(), ws.numel() * ws.element_size())


def route(cfg, x, w_router, topk_idx, gates, logit_bias=None, sel_bias=None, logits_in=None, logits=None,
          probsum=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _call("moe_route", ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(sel_bias),
          _ptr(logits_in), _ptr(logits), _ptr(topk_idx), _ptr(gates), _ptr(probsum), wp, wb, _stream(stream))


def permute(cfg, topk_idx, x, counts, offsets, perm, slot_pos, x_perm=None, drop_count=None, ws=None,
            stream=None):
    wp, wb = _ws(ws)
    _call("moe_permute", ctypes.byref(cfg), _ptr(topk_idx), _ptr(x), _ptr(counts), _ptr(offsets), _ptr(perm),
          _ptr(slot_pos), _ptr(drop_count), _ptr(x_perm), wp, wb, _stream(stream))


def permute_noalloc(cfg, topk_idx, x, counts, offsets, perm, slot_pos, x_perm=None, drop_count=None, stream=None):
    """moe_permute_noalloc: moe_permute on the library's static per-GPU scratch (no workspace)."""
    _call("moe_permute_noalloc", ctypes.byref(cfg), _ptr(topk_idx), _ptr(x), _ptr(counts), _ptr(offsets),
          _ptr(perm), _ptr(slot_pos), _ptr(drop_count), _ptr(x_perm), _stream(stream))


def expert_ffn(cfg, x_perm, offsets, w1, w3, w2, h_tmp, y_perm, b1=None, b2=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _call("moe_expert_ffn", ctypes.byref(cfg), _ptr(x_perm), _ptr(offsets), _ptr(w1), _ptr(w3), _ptr(w2),
          _ptr(b1), _ptr(b2), _ptr(h_tmp), _ptr(y_perm), wp, wb, _stream(stream))


def expert_up(cfg, x_perm, offsets, w1, w3, h_tmp, b1=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _call("moe_expert_up", ctypes.byref(cfg), _ptr(x_perm), _ptr(offsets), _ptr(w1), _ptr(w3), _ptr(b1),
          _ptr(h_tmp), wp, wb, _stream(stream))


def expert_up_gather(cfg, x, perm, offsets, w1, w3, h_tmp, b1=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _call("moe_expert_up_gather", ctypes.byref(cfg), _ptr(x), _ptr(perm), _ptr(offsets), _ptr(w1), _ptr(w3),
          _ptr(b1), _ptr(h_tmp), wp, wb, _stream(stream))


def expert_up_save(cfg, x, perm, offsets, w1, w3, h_tmp, pre_act, b1=None, ws=None, stream=None):
    """moe_expert_up_save: expert_up_gather that also writes the pre-activations [n, R, F] for backward()."""
    wp, wb = _ws(ws)
    _call("moe_expert_up_save", ctypes.byref(cfg), _ptr(x), _ptr(perm), _ptr(offsets), _ptr(w1), _ptr(w3),
          _ptr(b1), _ptr(h_tmp), _ptr(pre_act), wp, wb, _stream(stream))


def expert_down_combine(cfg, h_tmp, offsets, perm, slot_pos, gates, w2, out, b2=None, residual=None, shared_y=None,
                        ws=None, stream=None):
    """moe_expert_down_combine: top-1 down projection with the gate-weighted combine in its epilogue."""
    wp, wb = _ws(ws)
    _call("moe_expert_down_combine", ctypes.byref(cfg), _ptr(h_tmp), _ptr(offsets), _ptr(perm), _ptr(slot_pos),
          _ptr(gates), _ptr(w2), _ptr(b2), _ptr(residual), _ptr(shared_y), _ptr(out), wp, wb, _stream(stream))


def quantize_fp8(w, q, scales, stream=None):
    """Per-row E4M3 codes and fp32 scales of a bf16 matrix (rows = all leading dims)."""
    cols = int(w.shape[-1])
    rows = int(w.numel() // cols) if cols else 0
    _call("moe_quantize_fp8", _ptr(w), rows, cols, _ptr(q), _ptr(scales), _stream(stream))


def probe_hbm_read(buf, sink, stream=None):
    """moe_probe_hbm_read: one read of every byte of `buf` (a device tensor)."""
    _call("moe_probe_hbm_read", _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream))


def probe_mfma_bf16(operands, iters, sink, stream=None):
    """moe_probe_mfma_bf16: `iters` rounds of independent bf16 MFMAs on every wavefront of the chip."""
    _call("moe_probe_mfma_bf16", _ptr(operands), int(iters), _ptr(sink), _stream(stream))


def probe_mfma_flop_per_iter() -> int:
    n = c_int64(0)
    _call("moe_probe_mfma_flop_per_iter", ctypes.byref(n))
    return n.value


def expert_up_fp8(cfg, x, perm, offsets, w1q, w3q, s1, s3, h_tmp, b1=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _call("moe_expert_up_fp8", ctypes.byref(cfg), _ptr(x), _ptr(perm), _ptr(offsets), _ptr(w1q), _ptr(w3q),
          _ptr(s1), _ptr(s3), _ptr(b1), _ptr(h_tmp), wp, wb, _stream(stream))


def expert_down_fp8(cfg, h_tmp, offsets, w2q, s2, y_perm, b2=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _call("moe_expert_down_fp8", ctypes.byref(cfg), _ptr(h_tmp), _ptr(offsets), _ptr(w2q), _ptr(s2), _ptr(b2),
          _ptr(y_perm), wp, wb, _stream(stream))


def expert_down(cfg, h_tmp, offsets, w2, y_perm, b2=None, ws=None, stream=None):
    wp, wb = _ws(ws)
    _call("moe_expert_down", ctypes.byref(cfg), _ptr(h_tmp), _ptr(offsets), _ptr(w2), _ptr(b2), _ptr(y_perm),
          wp, wb, _stream(stream))


def shared_ffn(cfg, x, sh_w1, sh_w3, sh_w2, h_tmp, y_sh, ws=None, stream=None):
    wp, wb = _ws(ws)
    _call("moe_shared_ffn", ctypes.byref(cfg), _ptr(x), _ptr(sh_w1), _ptr(sh_w3), _ptr(sh_w2), _ptr(h_tmp),
          _ptr(y_sh), wp, wb, _stream(stream))


def combine(cfg, y_perm, slot_pos, gates, out, residual=None, shared_y=None, stream=None):
    _call("moe_combine", ctypes.byref(cfg), _ptr(y_perm), _ptr(slot_pos), _ptr(gates), _ptr(residual),
          _ptr(shared_y), _ptr(out), _stream(stream))


def bias_update(cfg, counts, gamma, sel_bias, signs=None, stream=None):
    _call("moe_bias_update", ctypes.byref(cfg), _ptr(counts), float(gamma), _ptr(sel_bias), _ptr(signs),
          _stream(stream))


def aux_loss(cfg, counts, probsum, aux, stream=None):
    _call("moe_aux_loss", ctypes.byref(cfg), _ptr(counts), _ptr(probsum), _ptr(aux), _stream(stream))


def forward(cfg, weights: dict, x, out, residual=None, sel_bias=None, outputs: dict | None = None,
            bias_gamma=0.0, ws=None, stream=None):
    """moe_forward.  ``weights``: w_router, logit_bias, w1, w3, w2, b1, b2, sh_w1, sh_w3, sh_w2
    (missing keys are NULL).  ``outputs``: optional tensors by moe_outputs field name."""
    W = MoeWeights(*[_ptr(weights.get(n)) for n, _ in MoeWeights._fields_])
    o = dict(outputs or {})
    o["out"] = out
    O = MoeOutputs(*[_ptr(o.get(n)) for n, _ in MoeOutputs._fields_[:-1]], float(bias_gamma))
    wp, wb = _ws(ws)
    _call("moe_forward", ctypes.byref(cfg), ctypes.byref(W), _ptr(x), _ptr(residual), _ptr(sel_bias),
          ctypes.byref(O), wp, wb, _stream(stream))


def backward_workspace_size(cfg: MoeConfig) -> int:
    n = c_size_t(0)
    _call("moe_backward_workspace_size", ctypes.byref(cfg), ctypes.byref(n))
    return n.value


def backward(cfg, weights: dict, x, dout, saved: dict, grads: dict, d_aux=0.0, ws=None, stream=None):
    """moe_backward: `weights` as for forward(); `saved` holds logits, topk_idx, gates, counts,
    offsets, perm, slot_pos, y_perm of the forward and optionally pre_act (from expert_up_save);
    `grads` the output tensors (see moe_grads)."""
    W = MoeWeights(*[_ptr(weights.get(n)) for n in ("w_router", "logit_bias", "w1", "w3", "w2", "b1", "b2",
                                                    "sh_w1", "sh_w3", "sh_w2")])
    S = MoeSaved(*[_ptr(saved.get(n)) for n in ("logits", "topk_idx", "gates", "counts", "offsets", "perm",
                                                "slot_pos", "y_perm", "pre_act")])
    G = MoeGrads(*[_ptr(grads.get(n)) for n in ("dx", "dw_router", "dlogit_bias", "dw1", "dw3", "dw2", "db1", "db2",
                                                "dsh_w1", "dsh_w3", "dsh_w2", "dgates")])
    wp, wb = _ws(ws)
    _call("moe_backward", ctypes.byref(cfg), ctypes.byref(W), _ptr(x), _ptr(dout), c_float(d_aux), ctypes.byref(S),
          ctypes.byref(G), wp, wb, _stream(stream))
