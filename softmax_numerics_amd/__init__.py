"""FP8 P-cast attention forward for AMD MI355X -- Python binding of libpcast_attn.so.

Argument marshalling only: every step of the attention runs in the HIP
kernels behind the C ABI declared in include/pcast_attn.h.  PyTorch provides
device memory and the stream.  There is no fallback: if the library is not
built, or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpcast_attn.so")

PCAST_OK, PCAST_EINVAL, PCAST_ENOTSUP, PCAST_EHIP = 0, 1, 2, 3
KV_BLOCK = 64
ORDERS = {"forward": 0, "reverse": 1, 0: 0, 1: 1}

# Every symbol include/pcast_attn.h declares.
EXPORTS = ("attn_fwd_pcast", "pcast_prepare_v", "attn_fwd_pcast_prepared", "pcast_stats_words",
           "pcast_workspace_bytes", "pcast_strerror", "pcast_abi_version", "pcast_workspace_bytes_qk8",
           "pcast_prepare_qk8", "attn_fwd_pcast_qk8_prepared", "attn_fwd_pcast_qk8",
           "attn_fwd_pcast_rows", "pcast_sink_max_mean", "pcast_delta_critical",
           "pcast_underflow_model", "pcast_lost_mass_model", "attn_decode_pcast",
           "pcast_decode_workspace_bytes", "attn_bwd_pcast", "pcast_bwd_workspace_bytes",
           "pcast_workspace_bytes_qk8_rot", "pcast_prepare_qk8_rot", "attn_fwd_pcast_qk8_rot_prepared",
           "attn_decode_pcast_qk8", "pcast_cast_e4m3", "pcast_collapse_check",
           "attn_fwd_pcast_noalloc", "attn_fwd_pcast_multi")

_lock = threading.Lock()
_lib = None


class PcastError(RuntimeError):
    def __init__(self, code: int, text: str):
        super().__init__(f"attn_fwd_pcast failed ({code}): {text}")
        self.code = code


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (raises if it is missing)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(f"{path} is not built; run __graft_entry__.build() or "
                                   "python -m softmax_numerics_amd.build")
            lib = ctypes.CDLL(path)
            P, I = ctypes.c_void_p, ctypes.c_int
            lib.attn_fwd_pcast.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_float, I, P, P, P]
            lib.attn_fwd_pcast.restype = I
            lib.attn_fwd_pcast_noalloc.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_float, I, P, P, P]
            lib.attn_fwd_pcast_noalloc.restype = I
            lib.attn_fwd_pcast_multi.argtypes = [P, P, P, I, I, I, I, I, I, I, P, P, P, P, P, P]
            lib.attn_fwd_pcast_multi.restype = I
            lib.pcast_prepare_v.argtypes = [P, I, I, I, I, ctypes.c_float, P, P]
            lib.pcast_prepare_v.restype = I
            lib.attn_fwd_pcast_prepared.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_float, I,
                                                    P, P, P]
            lib.attn_fwd_pcast_prepared.restype = I
            lib.pcast_stats_words.argtypes = [I, I, I]
            lib.pcast_stats_words.restype = ctypes.c_size_t
            lib.pcast_workspace_bytes.argtypes = [I, I, I, I, ctypes.c_float]
            lib.pcast_workspace_bytes.restype = ctypes.c_size_t
            lib.pcast_strerror.argtypes = [I]
            lib.pcast_strerror.restype = ctypes.c_char_p
            lib.pcast_abi_version.argtypes = []
            lib.pcast_abi_version.restype = I
            lib.pcast_workspace_bytes_qk8.argtypes = [I, I, I, I]
            lib.pcast_workspace_bytes_qk8.restype = ctypes.c_size_t
            lib.pcast_prepare_qk8.argtypes = [P, P, I, I, I, I, P, P]
            lib.pcast_prepare_qk8.restype = I
            lib.attn_fwd_pcast_qk8_prepared.argtypes = [P, P, P, I, I, I, I, I, I, ctypes.c_float, I, P, P,
                                                        P]
            lib.attn_fwd_pcast_qk8_prepared.restype = I
            lib.attn_fwd_pcast_qk8.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_float, I, P, P, P]
            lib.attn_fwd_pcast_qk8.restype = I
            lib.attn_fwd_pcast_rows.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_float, I, P, P, P, P, P]
            lib.attn_fwd_pcast_rows.restype = I
            lib.attn_decode_pcast.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_float, I, I, P, P, P, P]
            lib.attn_decode_pcast.restype = I
            lib.attn_decode_pcast_qk8.argtypes = [P, P, P, I, I, I, I, I, I, ctypes.c_float, I, I, P, P, P, P]
            lib.attn_decode_pcast_qk8.restype = I
            lib.pcast_decode_workspace_bytes.argtypes = [I, I, I, I, I]
            lib.pcast_decode_workspace_bytes.restype = ctypes.c_size_t
            lib.attn_bwd_pcast.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P]
            lib.attn_bwd_pcast.restype = I
            lib.pcast_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
            lib.pcast_bwd_workspace_bytes.restype = ctypes.c_size_t
            lib.pcast_workspace_bytes_qk8_rot.argtypes = [I, I, I, I, I]
            lib.pcast_workspace_bytes_qk8_rot.restype = ctypes.c_size_t
            lib.pcast_prepare_qk8_rot.argtypes = [P, P, P, P, I, I, I, I, I, P, P]
            lib.pcast_prepare_qk8_rot.restype = I
            lib.attn_fwd_pcast_qk8_rot_prepared.argtypes = [P, P, I, I, I, I, I, I, ctypes.c_float, I, P, P, P]
            lib.attn_fwd_pcast_qk8_rot_prepared.restype = I
            lib.pcast_cast_e4m3.argtypes = [P, P, ctypes.c_longlong, ctypes.c_float, P]
            lib.pcast_cast_e4m3.restype = I
            D = ctypes.c_double
            lib.pcast_sink_max_mean.argtypes = [I]
            lib.pcast_sink_max_mean.restype = D
            lib.pcast_delta_critical.argtypes = [D, I]
            lib.pcast_delta_critical.restype = D
            lib.pcast_underflow_model.argtypes = [D, D, I]
            lib.pcast_underflow_model.restype = D
            lib.pcast_lost_mass_model.argtypes = [D, D, I]
            lib.pcast_lost_mass_model.restype = D
            lib.pcast_collapse_check.argtypes = [P, I, D, I, P, P, P, P, P]
            lib.pcast_collapse_check.restype = I
            _lib = lib
    return _lib


def strerror(code: int) -> str:
    return load_library().pcast_strerror(code).decode()


def attn_fwd_pcast(Q, K, V, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats, stream) -> int:
    """Raw call with integer device addresses (0 for NULL); returns the C return code."""
    return int(load_library().attn_fwd_pcast(Q, K, V, bias or None, B, Hq, Hkv, N, d, int(causal),
                                             float(S), int(order), out, stats or None, stream or None))


NOALLOC_SCRATCH_BYTES = 64 << 20


def attn_fwd_pcast_noalloc(Q, K, V, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats, stream) -> int:
    """Raw attn_fwd_pcast_noalloc (no allocation; library scratch) with integer device addresses."""
    return int(load_library().attn_fwd_pcast_noalloc(Q, K, V, bias or None, B, Hq, Hkv, N, d, int(causal),
                                                     float(S), int(order), out, stats or None, stream or None))


def attn_fwd_pcast_multi(Q, K, workspace, B, Hq, Hkv, N, d, causal, biases, Ss, orders, outs, stats,
                         stream) -> int:
    """Raw attn_fwd_pcast_multi: integer device addresses; biases, outs and stats are lists of
    addresses (0 for NULL; stats None for no counting), Ss and orders lists of numbers."""
    n = len(Ss)
    ptrs = ctypes.c_void_p * n
    b_arr = ptrs(*[(x or None) for x in biases]) if biases is not None else None
    o_arr = ptrs(*outs)
    s_arr = ptrs(*stats) if stats is not None else None
    S_arr = (ctypes.c_float * n)(*[float(x) for x in Ss])
    r_arr = (ctypes.c_int * n)(*[int(x) for x in orders])
    return int(load_library().attn_fwd_pcast_multi(Q, K, workspace, B, Hq, Hkv, N, d, int(causal), n, b_arr, S_arr,
                                                   r_arr, o_arr, s_arr, stream or None))


def prepare_v(V, B, Hkv, N, d, S, workspace, stream) -> int:
    """Raw pcast_prepare_v with integer device addresses; returns the C return code."""
    return int(load_library().pcast_prepare_v(V, B, Hkv, N, d, float(S), workspace, stream or None))


def attn_fwd_pcast_prepared(Q, K, workspace, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats,
                            stream) -> int:
    """Raw attn_fwd_pcast_prepared with integer device addresses; returns the C return code."""
    return int(load_library().attn_fwd_pcast_prepared(
        Q, K, workspace, bias or None, B, Hq, Hkv, N, d, int(causal), float(S), int(order), out,
        stats or None, stream or None))


def attn_fwd_pcast_qk8(Q, K, V, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats, stream) -> int:
    """Raw attn_fwd_pcast_qk8 (FP8 logits) with integer device addresses; returns the C return code."""
    return int(load_library().attn_fwd_pcast_qk8(Q, K, V, bias or None, B, Hq, Hkv, N, d, int(causal),
                                                 float(S), int(order), out, stats or None, stream or None))


def prepare_qk8(K, V, B, Hkv, N, d, workspace, stream) -> int:
    """Raw pcast_prepare_qk8 with integer device addresses; returns the C return code."""
    return int(load_library().pcast_prepare_qk8(K, V, B, Hkv, N, d, workspace, stream or None))


def attn_fwd_pcast_qk8_prepared(Q, workspace, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats,
                                stream) -> int:
    """Raw attn_fwd_pcast_qk8_prepared with integer device addresses; returns the C return code."""
    return int(load_library().attn_fwd_pcast_qk8_prepared(
        Q, workspace, bias or None, B, Hq, Hkv, N, d, int(causal), float(S), int(order), out,
        stats or None, stream or None))


def attn_fwd_pcast_rows(Q, K, workspace, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats, lse, lost,
                        stream) -> int:
    """Raw attn_fwd_pcast_rows with integer device addresses (0 for NULL); returns the C return code."""
    return int(load_library().attn_fwd_pcast_rows(
        Q, K, workspace, bias or None, B, Hq, Hkv, N, d, int(causal), float(S), int(order), out,
        stats or None, lse or None, lost or None, stream or None))


def attn_decode_pcast(Q, K, vop, bias, B, Hq, Hkv, Nq, Nk, d, S, order, split_keys, out, stats, workspace,
                      stream) -> int:
    """Raw attn_decode_pcast with integer device addresses (0 for NULL); returns the C return code."""
    return int(load_library().attn_decode_pcast(
        Q, K, vop, bias or None, B, Hq, Hkv, Nq, Nk, d, float(S), int(order), int(split_keys), out,
        stats or None, workspace, stream or None))


def attn_decode_pcast_qk8(Q, qk8_workspace, bias, B, Hq, Hkv, Nq, Nk, d, S, order, split_keys, out, stats,
                          workspace, stream) -> int:
    """Raw attn_decode_pcast_qk8 with integer device addresses (0 for NULL); returns the C return code."""
    return int(load_library().attn_decode_pcast_qk8(
        Q, qk8_workspace, bias or None, B, Hq, Hkv, Nq, Nk, d, float(S), int(order), int(split_keys), out,
        stats or None, workspace, stream or None))


def decode_workspace_bytes(B: int, Hkv: int, Nk: int, d: int, split_keys: int) -> int:
    return int(load_library().pcast_decode_workspace_bytes(B, Hkv, Nk, d, split_keys))


def attn_bwd_pcast(Q, K, V, O, dO, lse, bias, B, Hq, Hkv, N, d, causal, dQ, dK, dV, workspace, stream) -> int:
    """Raw attn_bwd_pcast with integer device addresses (0 for NULL); returns the C return code."""
    return int(load_library().attn_bwd_pcast(Q, K, V, O, dO, lse, bias or None, B, Hq, Hkv, N, d, int(causal),
                                             dQ, dK, dV, workspace, stream or None))


def bwd_workspace_bytes(B: int, Hq: int, Hkv: int, N: int, d: int) -> int:
    return int(load_library().pcast_bwd_workspace_bytes(B, Hq, Hkv, N, d))


def sink_max_mean(k: int = 4) -> float:
    return float(load_library().pcast_sink_max_mean(int(k)))


def delta_critical(S: float, k: int = 4) -> float:
    """Sink strength above which forward order zeroes most non-sink codes at scale S."""
    return float(load_library().pcast_delta_critical(float(S), int(k)))


def underflow_model(delta: float, S: float, k: int = 4) -> float:
    return float(load_library().pcast_underflow_model(float(delta), float(S), int(k)))


def lost_mass_model(delta: float, S: float, k: int = 4) -> float:
    return float(load_library().pcast_lost_mass_model(float(delta), float(S), int(k)))


def collapse_check(bias, S: float, order="forward") -> dict:
    """The collapse model's verdict for a bias (numpy array or torch tensor, copied to
    the host): keys delta, k, delta_c, underflow, collapse (see pcast_collapse_check)."""
    import numpy as np

    if bias is not None and hasattr(bias, "detach"):
        bias = bias.detach().cpu().numpy()
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    if b is not None and b.ndim != 1:
        raise ValueError("bias must be 1-D")
    N = 1 if b is None else b.size
    delta, dc, under = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    k, col = ctypes.c_int(), ctypes.c_int()
    rc = load_library().pcast_collapse_check(None if b is None else b.ctypes.data, N, float(S), ORDERS[order],
                                             ctypes.byref(delta), ctypes.byref(k), ctypes.byref(dc),
                                             ctypes.byref(under), ctypes.byref(col))
    if rc != PCAST_OK:
        raise PcastError(rc, "pcast_collapse_check: bad arguments")
    return {"delta": delta.value, "k": k.value, "delta_c": dc.value, "underflow": under.value,
            "collapse": bool(col.value)}


def workspace_bytes_qk8_rot(B: int, Hq: int, Hkv: int, N: int, d: int) -> int:
    return int(load_library().pcast_workspace_bytes_qk8_rot(B, Hq, Hkv, N, d))


def prepare_qk8_rot(Q, K, V, signs, B, Hq, Hkv, N, d, workspace, stream) -> int:
    """Raw pcast_prepare_qk8_rot with integer device addresses; returns the C return code."""
    return int(load_library().pcast_prepare_qk8_rot(Q, K, V, signs, B, Hq, Hkv, N, d, workspace, stream or None))


def attn_fwd_pcast_qk8_rot_prepared(workspace, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats,
                                    stream) -> int:
    """Raw attn_fwd_pcast_qk8_rot_prepared with integer device addresses; returns the C return code."""
    return int(load_library().attn_fwd_pcast_qk8_rot_prepared(
        workspace, bias or None, B, Hq, Hkv, N, d, int(causal), float(S), int(order), out, stats or None,
        stream or None))


def cast_e4m3(P, codes, n, S, stream) -> int:
    """Raw pcast_cast_e4m3 with integer device addresses; returns the C return code."""
    return int(load_library().pcast_cast_e4m3(P, codes, int(n), float(S), stream or None))


def workspace_bytes_qk8(B: int, Hkv: int, N: int, d: int) -> int:
    return int(load_library().pcast_workspace_bytes_qk8(B, Hkv, N, d))


def stats_words(B: int, Hq: int, N: int) -> int:
    return int(load_library().pcast_stats_words(B, Hq, N))


def workspace_bytes(B: int, Hkv: int, N: int, d: int, S: float) -> int:
    return int(load_library().pcast_workspace_bytes(B, Hkv, N, d, float(S)))


def forward(q, k, v, bias=None, causal: bool = True, S: float = 256.0, order="reverse",
            stats: bool = False, out=None, qk_fp8: bool = False, check_collapse: bool = False):
    """O = softmax(q k^T / sqrt(d) + bias) v with the P-cast, on the current stream.

    q: bf16 [B, Hq, N, d]; k, v: bf16 [B, Hkv, N, d]; bias: fp32 [N] or None.
    S > 0: P*S cast to E4M3; S = 0: the bf16 reference path.  qk_fp8: Q and K
    rounded to E4M3 with power-of-two scales per query row and per 64-key
    block, logits on the FP8 matrix cores (needs S > 0).  out: an fp32
    [B, Hq, N, d] contiguous tensor on q's device to write into, or None.
    check_collapse: copy the bias to the host (a synchronisation) and warn when
    pcast_collapse_check predicts that the cast zeroes most non-sink
    probabilities.  Returns (out fp32 [B, Hq, N, d], stats int64
    [B, Hq, N/64, 2] or None).
    """
    import warnings

    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-D bfloat16 tensor on the GPU")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, N, d] matching q")
    if bias is not None and (bias.dtype != torch.float32 or not bias.is_cuda or bias.shape != (N,)
                             or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 [N] tensor on the GPU")
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
    elif (out.dtype != torch.float32 or out.device != q.device or tuple(out.shape) != (B, Hq, N, d)
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous float32 [B, Hq, N, d] tensor on q's device")
    if check_collapse and S > 0:
        r = collapse_check(bias, S, order)
        if r["collapse"]:
            warnings.warn(f"P-cast collapse predicted: sink strength {r['delta']:g} on {r['k']} keys exceeds "
                          f"Delta_c({S:g}) = {r['delta_c']:.3f} in forward order; about "
                          f"{100 * r['underflow']:.0f} % of the non-sink codes will be zero", RuntimeWarning)
    st = None
    if stats:
        st = torch.empty(stats_words(B, Hq, N), dtype=torch.int64, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    call = attn_fwd_pcast_qk8 if qk_fp8 else attn_fwd_pcast
    rc = call(q.data_ptr(), k.data_ptr(), v.data_ptr(), 0 if bias is None else bias.data_ptr(),
              B, Hq, Hkv, N, d, causal, S, ORDERS[order], out.data_ptr(),
              0 if st is None else st.data_ptr(), stream)
    if rc != PCAST_OK:
        raise PcastError(rc, strerror(rc))
    if st is not None:
        st = st.view(B, Hq, -1, 2)
    return out, st


def forward_multi(q, k, v, configs, causal: bool = True, stats: bool = False):
    """Several (bias, S, order) configurations of the forward on the same q, k, v in one
    launch per conversion mode (attn_fwd_pcast_multi).  configs: list of (bias fp32 [N]
    tensor or None, S > 0, order).  Returns (list of out, list of stats or None), each
    equal to forward() with that configuration."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-D bfloat16 tensor on the GPU")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, N, d] matching q")
    if not configs:
        raise ValueError("configs must not be empty")
    for bias, _, _ in configs:
        if bias is not None and (bias.dtype != torch.float32 or not bias.is_cuda or bias.shape != (N,)
                                 or not bias.is_contiguous()):
            raise ValueError("each bias must be a contiguous float32 [N] tensor on the GPU")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    ws = torch.empty(workspace_bytes(B, Hkv, N, d, 1.0), dtype=torch.uint8, device=q.device)
    rc = prepare_v(v.data_ptr(), B, Hkv, N, d, 1.0, ws.data_ptr(), stream)
    if rc != PCAST_OK:
        raise PcastError(rc, strerror(rc))
    outs = [torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device) for _ in configs]
    sts = [torch.empty(stats_words(B, Hq, N), dtype=torch.int64, device=q.device) for _ in configs] if stats else None
    rc = attn_fwd_pcast_multi(q.data_ptr(), k.data_ptr(), ws.data_ptr(), B, Hq, Hkv, N, d, causal,
                              [0 if c[0] is None else c[0].data_ptr() for c in configs],
                              [c[1] for c in configs], [ORDERS[c[2]] for c in configs],
                              [o.data_ptr() for o in outs], None if sts is None else [x.data_ptr() for x in sts],
                              stream)
    if rc != PCAST_OK:
        raise PcastError(rc, strerror(rc))
    return outs, (None if sts is None else [x.view(B, Hq, -1, 2) for x in sts])


_ATTENTION_FUNCTION = None


def _attention_function():
    """The torch.autograd.Function behind attention(), defined on first use (torch is
    imported lazily by this package)."""
    global _ATTENTION_FUNCTION
    if _ATTENTION_FUNCTION is not None:
        return _ATTENTION_FUNCTION
    import torch

    class PcastAttention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, bias, causal, S, order):
            _check_qkv(q, k, v, bias)
            if not S > 0:
                raise ValueError("attention() needs S > 0 (the P-cast path; its log-sum-exp feeds the backward)")
            B, Hq, N, d = q.shape
            Hkv = k.shape[1]
            stream = torch.cuda.current_stream(q.device).cuda_stream
            ws = torch.empty(workspace_bytes(B, Hkv, N, d, S), dtype=torch.uint8, device=q.device)
            out = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
            lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
            bp = 0 if bias is None else bias.data_ptr()
            rc = prepare_v(v.data_ptr(), B, Hkv, N, d, S, ws.data_ptr(), stream)
            if rc == PCAST_OK:
                # lost NULL: the pipelined forward writes out and lse alone
                rc = attn_fwd_pcast_rows(q.data_ptr(), k.data_ptr(), ws.data_ptr(), bp, B, Hq, Hkv, N, d, causal, S,
                                         ORDERS[order], out.data_ptr(), 0, lse.data_ptr(), 0, stream)
            if rc != PCAST_OK:
                raise PcastError(rc, strerror(rc))
            ctx.causal = bool(causal)
            ctx.has_bias = bias is not None
            ctx.save_for_backward(q, k, v, out, lse, *([bias] if bias is not None else []))
            return out

        @staticmethod
        def backward(ctx, grad_out):
            q, k, v, out, lse, *rest = ctx.saved_tensors
            bias = rest[0] if ctx.has_bias else None
            B, Hq, N, d = q.shape
            Hkv = k.shape[1]
            # the backward's C ABI takes dO in bf16 and writes fp32 gradients; the
            # conversions to and from the inputs' bf16 are torch's
            do = grad_out.to(torch.bfloat16).contiguous()
            dq = torch.empty((B, Hq, N, d), dtype=torch.float32, device=q.device)
            dk = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=q.device)
            dv = torch.empty_like(dk)
            wb = torch.empty(bwd_workspace_bytes(B, Hq, Hkv, N, d), dtype=torch.uint8, device=q.device)
            stream = torch.cuda.current_stream(q.device).cuda_stream
            rc = attn_bwd_pcast(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), do.data_ptr(),
                                lse.data_ptr(), 0 if bias is None else bias.data_ptr(), B, Hq, Hkv, N, d,
                                ctx.causal, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), wb.data_ptr(), stream)
            if rc != PCAST_OK:
                raise PcastError(rc, strerror(rc))
            return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None, None, None

    _ATTENTION_FUNCTION = PcastAttention
    return PcastAttention


def _check_qkv(q, k, v, bias):
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-D bfloat16 tensor on the GPU")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, N, d] matching q")
    if bias is not None and (bias.dtype != torch.float32 or not bias.is_cuda or bias.shape != (N,)
                             or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 [N] tensor on the GPU")


def attention(q, k, v, bias=None, causal: bool = True, S: float = 256.0, order="reverse"):
    """The P-cast forward as a differentiable torch operation (S > 0): out fp32
    [B, Hq, N, d].  The forward runs pcast_prepare_v and attn_fwd_pcast_rows (out and
    the log-sum-exp, no counters); the backward runs attn_bwd_pcast on the saved q, k,
    v, out and log-sum-exp, i.e. the gradients of exact attention taken at the
    forward's output (the cast itself has no gradient), with dO rounded to bf16 and
    the fp32 gradients rounded to the inputs' bf16 by torch.  Any N.  The bias gets no
    gradient."""
    return _attention_function().apply(q, k, v, bias, causal, float(S), order)
