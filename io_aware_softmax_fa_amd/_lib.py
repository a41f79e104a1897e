"""ctypes view of the C ABI declared in include/fa.h (marshalling only)."""
from __future__ import annotations

import ctypes
import os
import threading

# FA_LIBRARY selects another build of the same library (a measurement variant
# from build.py); there is no fallback either way
LIB_PATH = os.environ.get("FA_LIBRARY") or \
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_fwd.so")

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_LAUNCH = -3
FA_ERR_TOO_LARGE = -4
FA_NOALLOC_SCRATCH_BYTES = 16 << 20

FA_F16 = 0
FA_BF16 = 1
FA_FP8_E4M3 = 2

_lock = threading.Lock()
_lib = None


class FaError(RuntimeError):
    def __init__(self, code: int, fn: str):
        self.code = code
        super().__init__(f"{fn} returned {code}: {strerror(code)}")


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m io_aware_softmax_fa_amd.build` (hipcc, gfx950)")
                h = ctypes.CDLL(LIB_PATH)
                vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
                h.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
                h.fa_fwd.restype = i
                h.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, f, f, f, i, i, i, i, f, i, vp]
                h.fa_fwd_fp8.restype = i
                h.fa_bwd.argtypes = [vp] * 10 + [i, i, i, i, f, i, i, vp]
                h.fa_bwd.restype = i
                h.fa_fwd_kv.argtypes = [vp] * 5 + [i] * 6 + [f, i, i, i, vp, vp]
                h.fa_fwd_kv.restype = i
                h.fa_fwd_kv_noalloc.argtypes = [vp] * 5 + [i] * 6 + [f, i, i, i, vp]
                h.fa_fwd_kv_noalloc.restype = i
                h.fa_fwd_kv_workspace.argtypes = [i, i, i, i, i]
                h.fa_fwd_kv_workspace.restype = ctypes.c_size_t
                h.fa_fwd_fp8_block.argtypes = [vp] * 8 + [i] * 4 + [f, i, vp]
                h.fa_fwd_fp8_block.restype = i
                h.fa_quantize_fp8.argtypes = [vp] * 4 + [i] * 6 + [vp]
                h.fa_quantize_fp8.restype = i
                h.fa_fwd_varlen.argtypes = [vp] * 8 + [i] * 8 + [f, i, i, i, vp, vp]
                h.fa_fwd_varlen.restype = i
                h.fa_varlen_order.argtypes = [vp, vp] + [i] * 6 + [vp, vp]
                h.fa_varlen_order.restype = i
                h.fa_fwd_varlen_workspace.argtypes = [i, i, i, i]
                h.fa_fwd_varlen_workspace.restype = ctypes.c_size_t
                h.fa_strerror.argtypes = [i]
                h.fa_strerror.restype = ctypes.c_char_p
                h.fa_version.argtypes = []
                h.fa_version.restype = i
                _lib = h
    return _lib


def strerror(code: int) -> str:
    return lib().fa_strerror(int(code)).decode()


def version() -> int:
    return int(lib().fa_version())


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream) -> int:
    """Raw call: pointers as ints, returns the C return code."""
    return int(lib().fa_fwd(q, k, v, o, lse, int(B), int(H), int(N), int(d), float(scale),
                            int(causal), int(dtype), stream))


def fa_fwd_fp8(q, k, v, o, lse, q_descale, k_descale, v_descale, B, H, N, d, scale, causal,
               stream) -> int:
    return int(lib().fa_fwd_fp8(q, k, v, o, lse, float(q_descale), float(k_descale),
                                float(v_descale), int(B), int(H), int(N), int(d), float(scale),
                                int(causal), stream))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, d, scale, causal, dtype,
           stream) -> int:
    return int(lib().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, int(B), int(H), int(N),
                            int(d), float(scale), int(causal), int(dtype), stream))


def fa_fwd_kv(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, dtype, num_splits, workspace,
              stream) -> int:
    return int(lib().fa_fwd_kv(q, k, v, o, lse, int(B), int(H), int(Hkv), int(Nq), int(Nk), int(d),
                               float(scale), int(causal), int(dtype), int(num_splits), workspace,
                               stream))


def fa_fwd_kv_noalloc(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, dtype, num_splits,
                      stream) -> int:
    return int(lib().fa_fwd_kv_noalloc(q, k, v, o, lse, int(B), int(H), int(Hkv), int(Nq), int(Nk),
                                       int(d), float(scale), int(causal), int(dtype),
                                       int(num_splits), stream))


def fa_fwd_kv_workspace(B, H, Nq, d, num_splits) -> int:
    return int(lib().fa_fwd_kv_workspace(int(B), int(H), int(Nq), int(d), int(num_splits)))


def fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, order, B, H, Hkv, max_q, max_k, total_q, total_k,
                  d, scale, causal, dtype, num_splits, workspace, stream) -> int:
    return int(lib().fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, order, int(B), int(H), int(Hkv),
                                   int(max_q), int(max_k), int(total_q), int(total_k), int(d),
                                   float(scale), int(causal), int(dtype), int(num_splits),
                                   workspace, stream))


def fa_varlen_order(cu_q, cu_k, B, max_q, max_k, total_q, total_k, num_splits, order,
                    stream) -> int:
    return int(lib().fa_varlen_order(cu_q, cu_k, int(B), int(max_q), int(max_k), int(total_q),
                                     int(total_k), int(num_splits), order, stream))


def fa_fwd_varlen_workspace(total_q, H, d, num_splits) -> int:
    return int(lib().fa_fwd_varlen_workspace(int(total_q), int(H), int(d), int(num_splits)))


def fa_fwd_fp8_block(q, k, v, o, lse, q_scale, k_scale, v_scale, B, H, N, d, scale, causal,
                     stream) -> int:
    return int(lib().fa_fwd_fp8_block(q, k, v, o, lse, q_scale, k_scale, v_scale, int(B), int(H),
                                      int(N), int(d), float(scale), int(causal), stream))


def fa_quantize_fp8(x, x8, scales, signs, B, H, N, d, block_rows, dtype, stream) -> int:
    return int(lib().fa_quantize_fp8(x, x8, scales, signs, int(B), int(H), int(N), int(d),
                                     int(block_rows), int(dtype), stream))
