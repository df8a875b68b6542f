"""ctypes binding of libmoe (the C ABI in include/moe.h).

Argument marshalling only: every function takes device tensors (or None), passes their data
pointers and the current HIP stream to the C entry point of the same name, and raises MoEError on a
non-zero status.  Nothing here computes any part of the layer.  Loading fails loudly when the
library has not been built (``python -m sparse_mixture_experts_counting_amd.build``).
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
GATE_SOFTMAX_TOPK, GATE_SOFTMAX_ALL, GATE_SIGMOID_TOPK = 0, 1, 2
ROUTE_LOGITS_IN = 0x1
EC_SCORES_IN = 0x1
STATUS = {0: "MOE_OK", 1: "MOE_ERR_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
          4: "MOE_ERR_DEVICE"}

EXPORTS = ("moe_workspace_bytes", "moe_status_str", "moe_route", "moe_dispatch", "moe_expert_ffn",
           "moe_expert_up", "moe_expert_down", "moe_combine", "moe_aux_loss",
           "moe_update_select_bias", "moe_transpose", "moe_backward_workspace_bytes",
           "moe_combine_backward", "moe_expert_backward", "moe_route_backward",
           "moe_expert_choice", "moe_gathered_workspace_bytes", "moe_expert_ffn_gathered",
           "moe_reroute", "moe_q_workspace_bytes", "moe_quantize_weights", "moe_expert_ffn_q",
           "moe_expert_ffn_save", "moe_expert_backward_saved", "moe_peak_mfma",
           "moe_peak_copy", "moe_dispatch_noalloc")


class MoEError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s" % (fn, msg))
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError("libmoe.so is not built at %s; run "
                      "`python -m sparse_mixture_experts_counting_amd.build`" % LIB_PATH)
_lib = ctypes.CDLL(LIB_PATH)

_p, _i, _u, _sz, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t, ctypes.c_float
_lib.moe_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
_lib.moe_workspace_bytes.restype = _sz
_lib.moe_status_str.argtypes = [_i]
_lib.moe_status_str.restype = ctypes.c_char_p
_lib.moe_route.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _u, _p, _p, _p, _p, _p, _p, _sz,
                          _p]
_lib.moe_dispatch.argtypes = [_p, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz, _p]
_lib.moe_expert_ffn.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _i, _p, _p, _sz, _p]
_lib.moe_expert_ffn_save.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _i, _p, _p, _p,
                                     _sz, _p]
_lib.moe_expert_backward_saved.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _i,
                                           _p, _p, _p, _p, _p, _sz, _p]
_lib.moe_expert_up.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _i, _p, _p, _sz, _p]
_lib.moe_expert_down.argtypes = [_p, _p, _i, _i, _i, _i, _i, _p, _i, _p, _p, _sz, _p]
_lib.moe_combine.argtypes = [_p, _p, _p, _i, _i, _i, _i, _p, _p, _p]
_lib.moe_aux_loss.argtypes = [_p, _p, _p, _i, _i, _i, _f, _f, _p, _p, _p]
_lib.moe_transpose.argtypes = [_p, _i, _i, _i, _i, _p, _p]
_lib.moe_update_select_bias.argtypes = [_p, _i, _i, _i, _f, _p, _p]
_lib.moe_backward_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
_lib.moe_backward_workspace_bytes.restype = _sz
_lib.moe_combine_backward.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _p, _p, _p]
_lib.moe_expert_backward.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _i, _p, _p,
                                     _p, _p, _p, _sz, _p]
_lib.moe_route_backward.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _f,
                                    _p, _p, _p, _p, _p, _sz, _p]
_lib.moe_expert_choice.argtypes = [_p, _i, _i, _i, _u, _p, _p, _p, _p, _p, _p]
_lib.moe_q_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
_lib.moe_q_workspace_bytes.restype = _sz
_lib.moe_quantize_weights.argtypes = [_p, _i, _i, _i, _i, _i, _p, _p, _p]
_lib.moe_expert_ffn_q.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _i,
                                  _p, _p, _sz, _p]
_lib.moe_reroute.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p,
                             _p, _sz, _p]
_lib.moe_gathered_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
_lib.moe_gathered_workspace_bytes.restype = _sz
_lib.moe_expert_ffn_gathered.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _i, _p, _p,
                                         _sz, _p]
_lib.moe_dispatch_noalloc.argtypes = [_p, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p]
_lib.moe_peak_mfma.argtypes = [_p, _i, _i, _p, _p]
_lib.moe_peak_copy.argtypes = [_p, _p, _sz, _p]
for _n in ("moe_dispatch_noalloc", "moe_peak_mfma", "moe_peak_copy", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_expert_up", "moe_expert_down",
           "moe_combine", "moe_aux_loss", "moe_transpose", "moe_update_select_bias",
           "moe_combine_backward", "moe_expert_backward", "moe_route_backward",
           "moe_expert_choice", "moe_expert_ffn_gathered", "moe_reroute",
           "moe_quantize_weights", "moe_expert_ffn_q"):
    getattr(_lib, _n).restype = _i
# Every exported entry point has its argument types declared (a missing declaration would pass
# 64-bit pointers and sizes as C ints).
for _n in EXPORTS:
    assert getattr(_lib, _n).argtypes is not None, _n


def lib():
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status):
    if status != 0:
        raise MoEError(fn, status, _lib.moe_status_str(status).decode())


def dtype_code(t):
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError("unsupported layer dtype %s" % t.dtype)


def workspace_bytes(T, d, d_ff, E, k, dt):
    return int(_lib.moe_workspace_bytes(T, d, d_ff, E, k, dt))


def route(x, w_r, logit_bias, T, d, E, k, dt, gating, flags, logits, topk_idx, topk_gate,
          prob_sum, lse_sq_sum, workspace, stream=None, select_bias=None):
    _check("moe_route", _lib.moe_route(
        _ptr(x), _ptr(w_r), _ptr(logit_bias), _ptr(select_bias), T, d, E, k, dt, gating, flags,
        _ptr(logits),
        _ptr(topk_idx), _ptr(topk_gate), _ptr(prob_sum), _ptr(lse_sq_sum), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))


def dispatch(topk_idx, T, E, k, capacity, counts, offsets, perm, inv, n_dropped, workspace,
             stream=None):
    _check("moe_dispatch", _lib.moe_dispatch(
        _ptr(topk_idx), T, E, k, capacity, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv),
        _ptr(n_dropped), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def dispatch_noalloc(topk_idx, T, E, k, capacity, counts, offsets, perm, inv, n_dropped,
                     stream=None):
    _check("moe_dispatch_noalloc", _lib.moe_dispatch_noalloc(
        _ptr(topk_idx), T, E, k, capacity, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv),
        _ptr(n_dropped), _stream(stream)))


def expert_ffn(x, perm, offsets, T, d, d_ff, E, k, w1, w3, w2, dt, out, workspace, stream=None):
    _check("moe_expert_ffn", _lib.moe_expert_ffn(
        _ptr(x), _ptr(perm), _ptr(offsets), T, d, d_ff, E, k, _ptr(w1), _ptr(w3), _ptr(w2), dt,
        _ptr(out), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def expert_ffn_save(x, perm, offsets, T, d, d_ff, E, k, w1, w3, w2, dt, out, saved, workspace,
                    stream=None):
    _check("moe_expert_ffn_save", _lib.moe_expert_ffn_save(
        _ptr(x), _ptr(perm), _ptr(offsets), T, d, d_ff, E, k, _ptr(w1), _ptr(w3), _ptr(w2), dt,
        _ptr(out), _ptr(saved), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def expert_up(x, perm, offsets, T, d, d_ff, E, k, w1, w3, dt, h, workspace, stream=None):
    _check("moe_expert_up", _lib.moe_expert_up(
        _ptr(x), _ptr(perm), _ptr(offsets), T, d, d_ff, E, k, _ptr(w1), _ptr(w3), dt, _ptr(h),
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def expert_down(h, offsets, T, d, d_ff, E, k, w2, dt, out, workspace, stream=None):
    _check("moe_expert_down", _lib.moe_expert_down(
        _ptr(h), _ptr(offsets), T, d, d_ff, E, k, _ptr(w2), dt, _ptr(out), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))


def combine(expert_out, inv, topk_gate, T, d, k, dt, shared_out, y, stream=None):
    _check("moe_combine", _lib.moe_combine(
        _ptr(expert_out), _ptr(inv), _ptr(topk_gate), T, d, k, dt, _ptr(shared_out), _ptr(y),
        _stream(stream)))


def aux_loss(counts, prob_sum, lse_sq_sum, T, E, k, alpha, beta, aux, z, stream=None):
    _check("moe_aux_loss", _lib.moe_aux_loss(
        _ptr(counts), _ptr(prob_sum), _ptr(lse_sq_sum), T, E, k, float(alpha), float(beta),
        _ptr(aux), _ptr(z), _stream(stream)))


def transpose(src, batch, rows, cols, dt, dst, stream=None):
    """dst[b][c][r] = src[b][r][c] (weight layout conversion, at load time)."""
    _check("moe_transpose", _lib.moe_transpose(_ptr(src), batch, rows, cols, dt, _ptr(dst),
                                               _stream(stream)))


def update_select_bias(counts, T, E, k, rate, select_bias, stream=None):
    """select_bias[e] += rate * sign(T*k - E*counts[e]) (aux-loss-free balancing step)."""
    _check("moe_update_select_bias", _lib.moe_update_select_bias(
        _ptr(counts), T, E, k, float(rate), _ptr(select_bias), _stream(stream)))


def backward_workspace_bytes(T, d, d_ff, E, k, dt):
    return int(_lib.moe_backward_workspace_bytes(T, d, d_ff, E, k, dt))


def combine_backward(dy, expert_out, inv, topk_gate, T, d, k, dt, d_out, d_gate, stream=None):
    _check("moe_combine_backward", _lib.moe_combine_backward(
        _ptr(dy), _ptr(expert_out), _ptr(inv), _ptr(topk_gate), T, d, k, dt, _ptr(d_out),
        _ptr(d_gate), _stream(stream)))


def expert_backward(x, perm, offsets, T, d, d_ff, E, k, w1, w3, w2, d_out, dt, dx_rows, dw1, dw3,
                    dw2, workspace, stream=None):
    _check("moe_expert_backward", _lib.moe_expert_backward(
        _ptr(x), _ptr(perm), _ptr(offsets), T, d, d_ff, E, k, _ptr(w1), _ptr(w3), _ptr(w2),
        _ptr(d_out), dt, _ptr(dx_rows), _ptr(dw1), _ptr(dw3), _ptr(dw2), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))


def expert_backward_saved(saved, x, perm, offsets, T, d, d_ff, E, k, w1, w3, w2, d_out, dt,
                          dx_rows, dw1, dw3, dw2, workspace, stream=None):
    _check("moe_expert_backward_saved", _lib.moe_expert_backward_saved(
        _ptr(saved), _ptr(x), _ptr(perm), _ptr(offsets), T, d, d_ff, E, k, _ptr(w1), _ptr(w3),
        _ptr(w2), _ptr(d_out), dt, _ptr(dx_rows), _ptr(dw1), _ptr(dw3), _ptr(dw2),
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def route_backward(x, w_r, logits, topk_idx, topk_gate, d_gate, counts, T, d, E, k, dt, gating,
                   alpha, beta, dx_add, d_logits, dw_r, dx, workspace, stream=None):
    _check("moe_route_backward", _lib.moe_route_backward(
        _ptr(x), _ptr(w_r), _ptr(logits), _ptr(topk_idx), _ptr(topk_gate), _ptr(d_gate),
        _ptr(counts), T, d, E, k, dt, gating, float(alpha), float(beta), _ptr(dx_add),
        _ptr(d_logits), _ptr(dw_r), _ptr(dx), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))


def expert_choice(logits, T, E, C, flags, scores, offsets, perm, gate, slot, stream=None):
    _check("moe_expert_choice", _lib.moe_expert_choice(
        _ptr(logits), T, E, C, flags, _ptr(scores), _ptr(offsets), _ptr(perm), _ptr(gate),
        _ptr(slot), _stream(stream)))


def gathered_workspace_bytes(rows_max, d, d_ff, E, dt):
    return int(_lib.moe_gathered_workspace_bytes(rows_max, d, d_ff, E, dt))


def expert_ffn_gathered(x, rows, offsets, T, d, d_ff, E, rows_max, w1, w3, w2, dt, out, workspace,
                        stream=None):
    _check("moe_expert_ffn_gathered", _lib.moe_expert_ffn_gathered(
        _ptr(x), _ptr(rows), _ptr(offsets), T, d, d_ff, E, rows_max, _ptr(w1), _ptr(w3), _ptr(w2),
        dt, _ptr(out), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def reroute(logits, select_bias, topk_idx, topk_gate, offsets, inv, T, E, k, capacity, gating,
            topk_idx2, topk_gate2, offsets2, perm2, inv2, n_dropped2, workspace, stream=None):
    _check("moe_reroute", _lib.moe_reroute(
        _ptr(logits), _ptr(select_bias), _ptr(topk_idx), _ptr(topk_gate), _ptr(offsets), _ptr(inv),
        T, E, k, capacity, gating, _ptr(topk_idx2), _ptr(topk_gate2), _ptr(offsets2), _ptr(perm2),
        _ptr(inv2), _ptr(n_dropped2), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def q_workspace_bytes(T, d, d_ff, E, k, bits):
    return int(_lib.moe_q_workspace_bytes(T, d, d_ff, E, k, bits))


def quantize_weights(w, batch, rows, cols, dt, bits, q, scale, stream=None):
    """Per-row symmetric INT8 / INT4 quantization of bf16 weights (load time)."""
    _check("moe_quantize_weights", _lib.moe_quantize_weights(
        _ptr(w), batch, rows, cols, dt, bits, _ptr(q), _ptr(scale), _stream(stream)))


def expert_ffn_q(x, perm, offsets, T, d, d_ff, E, k, bits, q1, s1, q3, s3, q2, s2, dt, out,
                 workspace, stream=None):
    _check("moe_expert_ffn_q", _lib.moe_expert_ffn_q(
        _ptr(x), _ptr(perm), _ptr(offsets), T, d, d_ff, E, k, bits, _ptr(q1), _ptr(s1), _ptr(q3),
        _ptr(s3), _ptr(q2), _ptr(s2), dt, _ptr(out), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))


def peak_mfma(operands, blocks, iters, out, stream=None):
    _check("moe_peak_mfma", _lib.moe_peak_mfma(_ptr(operands), blocks, iters, _ptr(out),
                                               _stream(stream)))


def peak_copy(src, dst, nbytes, stream=None):
    _check("moe_peak_copy", _lib.moe_peak_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))
