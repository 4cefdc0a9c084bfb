"""ctypes binding of libdomino_mi355x.so: the same calls as include/domino.h, argument
marshalling only (tensors → device pointers, streams → hipStream_t handles, status →
exception). Every step of the layer runs in the library's HIP kernels; there is no
fallback path: if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

LIB_NAME = "libdomino_mi355x.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

# Mirrors of the header's enums and descriptor structs.
DOMINO_F32, DOMINO_BF16 = 0, 1
DOMINO_ACT_GELU_TANH, DOMINO_ACT_SWIGLU = 0, 1
DOMINO_MAX_PARTIALS = 16
STATUS_NAMES = {0: "DOMINO_OK", 1: "DOMINO_ERR_INVALID_ARG", 2: "DOMINO_ERR_SHAPE", 3: "DOMINO_ERR_ALIGN",
                4: "DOMINO_ERR_UNSUPPORTED", 5: "DOMINO_ERR_HIP"}
KERNEL_KINDS = {"reduce": 0, "fwd_gemm1": 1, "fwd_gemm2": 2, "dgrad_b": 3, "dgrad_a": 4, "wgrad_b": 5,
                "wgrad_a": 6, "qkv": 7, "attn": 8, "outproj": 9, "aux": 10, "attn_bwd_dkdv": 11, "outproj_dgrad": 12,
                "qkv_dgrad": 13, "outproj_wgrad": 14, "qkv_wgrad": 15, "attn_bwd_dq": 16, "attn_bwd_prep": 17,
                "group_fwd": 18, "group_bwd": 19,
                "bias_grad": 20}

# Every symbol the header declares (checked by the CPU export test).
EXPORTED = ("shard_reduce", "domino_block_fwd", "domino_block_fwd_workspace_size", "domino_block_bwd",
            "domino_block_bwd_noalloc",
            "domino_block_bwd_workspace_size", "domino_attn_block_fwd", "domino_attn_block_fwd_workspace_size",
            "domino_attn_block_bwd", "domino_attn_block_bwd_workspace_size",
            "domino_resid_ln_fwd", "domino_resid_ln_bwd", "domino_resid_ln_bwd_workspace_size", "domino_stack_fwd",
            "domino_stack_bwd", "domino_stack_bwd_workspace_size",
            "domino_status_string", "domino_last_error", "domino_timing_enable",
            "domino_timing_read", "domino_timing_kernel")


class MlpDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("ffn_shard", ctypes.c_int64), ("act", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("row_chunks", ctypes.c_int32), ("col_chunks", ctypes.c_int32), ("n_partials", ctypes.c_int32),
                ("no_join", ctypes.c_int32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("heads", ctypes.c_int64), ("head_dim", ctypes.c_int64), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("row_chunks", ctypes.c_int32), ("n_partials", ctypes.c_int32),
                ("no_join", ctypes.c_int32)]


class GroupDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("hidden", ctypes.c_int64), ("eps", ctypes.c_float),
                ("p_drop", ctypes.c_float)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("heads", ctypes.c_int64), ("head_dim", ctypes.c_int64), ("ffn_shard", ctypes.c_int64),
                ("act", ctypes.c_int32), ("eps", ctypes.c_float), ("p_drop", ctypes.c_float), ("scale", ctypes.c_float),
                ("row_chunks", ctypes.c_int32), ("n_partials", ctypes.c_int32), ("layers", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_VP = ctypes.c_void_p


class LayerParams(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("ln1_gamma", "ln1_beta", "A_qkv_s", "B_o_s", "b_o", "ln2_gamma", "ln2_beta", "A_s",
                                   "B_s", "b_2", "keep_attn", "keep_mlp", "b_qkv", "b_1")]


class LayerActs(ctypes.Structure):
    _fields_ = [("x_in", _VP), ("ln1", _VP), ("mean1", _VP), ("rstd1", _VP), ("QKV", _VP), ("O", _VP), ("lse", _VP),
                ("y_attn_own", _VP), ("peer_y_attn", ctypes.POINTER(_VP)), ("y_attn", _VP), ("h", _VP), ("ln2", _VP),
                ("mean2", _VP), ("rstd2", _VP), ("Hpre", _VP), ("H", _VP), ("y_mlp_own", _VP),
                ("peer_y_mlp", ctypes.POINTER(_VP)), ("y_mlp", _VP)]


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("d_ln1_gamma", "d_ln1_beta", "dA_qkv_s", "dB_o_s", "d_b_o", "d_ln2_gamma",
                                   "d_ln2_beta", "dA_s", "dB_s", "d_b_2", "d_x_in", "d_ym", "dHpre", "dx_mlp_own")] + \
        [("peer_dx_mlp", ctypes.POINTER(_VP))] + [(n, _VP) for n in ("dx_mlp", "d_h", "d_ya", "dO", "dQKV",
                                                                    "dx_attn_own")] + \
        [("peer_dx_attn", ctypes.POINTER(_VP)), ("dx_attn", _VP), ("d_b_qkv", _VP), ("d_b_1", _VP)]


class DominoError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with tensor_transformer_block_domino_amd.build.build()")
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    pp = ctypes.POINTER(ctypes.c_void_p)
    lib.shard_reduce.argtypes = [vp, i64, pp, i32, i64, i64, i64, i32, vp]
    lib.shard_reduce.restype = i32
    lib.domino_block_fwd.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, vp, vp, vp, vp, pp, vp, vp,
                                     ctypes.c_size_t, vp, vp]
    lib.domino_block_fwd.restype = i32
    for name, desc in (("domino_block_fwd_workspace_size", MlpDesc), ("domino_block_bwd_workspace_size", MlpDesc),
                       ("domino_attn_block_fwd_workspace_size", AttnDesc),
                       ("domino_attn_block_bwd_workspace_size", AttnDesc)):
        getattr(lib, name).argtypes = [ctypes.POINTER(desc)]
        getattr(lib, name).restype = ctypes.c_size_t
    lib.domino_block_bwd.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, vp, vp, vp, vp, vp, pp, vp, vp, vp, vp,
                                     i32, vp, ctypes.c_size_t, vp, vp]
    lib.domino_block_bwd.restype = i32
    lib.domino_block_bwd_noalloc.argtypes = [ctypes.POINTER(MlpDesc), vp, vp, vp, vp, vp, vp, vp, vp, pp, vp, vp, vp,
                                             vp, i32, vp, vp]
    lib.domino_block_bwd_noalloc.restype = i32
    lib.domino_attn_block_fwd.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp, pp, vp, vp,
                                          ctypes.c_size_t, vp, vp]
    lib.domino_attn_block_fwd.restype = i32
    lib.domino_attn_block_bwd.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, pp, vp,
                                          vp, vp, vp, i32, vp, ctypes.c_size_t, vp, vp]
    lib.domino_attn_block_bwd.restype = i32
    lib.domino_resid_ln_fwd.argtypes = [ctypes.POINTER(GroupDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.domino_resid_ln_fwd.restype = i32
    lib.domino_resid_ln_bwd.argtypes = [ctypes.POINTER(GroupDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        i32, vp, ctypes.c_size_t, vp]
    lib.domino_resid_ln_bwd.restype = i32
    lib.domino_resid_ln_bwd_workspace_size.argtypes = [ctypes.POINTER(GroupDesc)]
    lib.domino_resid_ln_bwd_workspace_size.restype = ctypes.c_size_t
    lib.domino_stack_fwd.argtypes = [ctypes.POINTER(LayerDesc), vp, ctypes.POINTER(LayerParams),
                                     ctypes.POINTER(LayerActs), vp, vp, ctypes.c_size_t, vp, vp]
    lib.domino_stack_fwd.restype = i32
    lib.domino_stack_bwd.argtypes = [ctypes.POINTER(LayerDesc), vp, ctypes.POINTER(LayerParams),
                                     ctypes.POINTER(LayerActs), ctypes.POINTER(LayerGrads), vp, vp, i32, vp,
                                     ctypes.c_size_t, vp, vp]
    lib.domino_stack_bwd.restype = i32
    lib.domino_stack_bwd_workspace_size.argtypes = [ctypes.POINTER(LayerDesc)]
    lib.domino_stack_bwd_workspace_size.restype = ctypes.c_size_t
    lib.domino_status_string.argtypes = [i32]
    lib.domino_status_string.restype = ctypes.c_char_p
    lib.domino_last_error.argtypes = []
    lib.domino_last_error.restype = ctypes.c_char_p
    lib.domino_timing_enable.argtypes = [i32]
    lib.domino_timing_enable.restype = i32
    lib.domino_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
    lib.domino_timing_read.restype = i32
    lib.domino_timing_kernel.argtypes = [i32, ctypes.c_char_p, ctypes.c_size_t]
    lib.domino_timing_kernel.restype = i32
    _lib = lib
    return lib


# ---------------------------------------------------------------------------------------
# Marshalling.
# ---------------------------------------------------------------------------------------
def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _ptr_array(items: Optional[Sequence]):
    if items is None:
        return None
    arr = (ctypes.c_void_p * max(1, len(items)))()
    for i, t in enumerate(items):
        arr[i] = _ptr(t)
    return arr


def _check(status: int):
    if status != 0:
        raise DominoError(status, load().domino_last_error().decode())


def shard_reduce(out, ld_out: int, partials: Sequence, ld_in: int, rows: int, cols: int, dtype: int, stream=None):
    _check(load().shard_reduce(_ptr(out), ld_out, _ptr_array(partials), len(partials), ld_in, rows, cols, dtype,
                               _stream(stream)))


def domino_block_fwd(desc: MlpDesc, X, A_s, B_s, Hpre, H, Y_own, peer_Y, Y, workspace=None, workspace_bytes: int = 0,
                     compute=None, comm=None, b1_s=None):
    _check(load().domino_block_fwd(ctypes.byref(desc), _ptr(X), _ptr(A_s), _ptr(B_s), _ptr(b1_s), _ptr(Hpre), _ptr(H),
                                   _ptr(Y_own), _ptr_array(peer_Y), _ptr(Y), _ptr(workspace), int(workspace_bytes),
                                   _stream(compute), _stream(comm)))


def domino_block_fwd_workspace_size(desc: MlpDesc) -> int:
    return int(load().domino_block_fwd_workspace_size(ctypes.byref(desc)))


def domino_block_bwd_workspace_size(desc: MlpDesc) -> int:
    return int(load().domino_block_bwd_workspace_size(ctypes.byref(desc)))


def domino_block_bwd_noalloc(desc: MlpDesc, X, A_s, B_s, Hpre, H, dY, dHpre, dX_own, peer_dX, dX, dA_s, dB_s,
                             accumulate: int = 0, compute=None, comm=None, d_b1_s=None):
    _check(load().domino_block_bwd_noalloc(ctypes.byref(desc), _ptr(X), _ptr(A_s), _ptr(B_s), _ptr(Hpre), _ptr(H),
                                           _ptr(dY), _ptr(dHpre), _ptr(dX_own), _ptr_array(peer_dX), _ptr(dX),
                                           _ptr(dA_s), _ptr(dB_s), _ptr(d_b1_s), int(accumulate), _stream(compute),
                                           _stream(comm)))


NOALLOC_SCRATCH_BYTES = 64 << 20   # DOMINO_NOALLOC_SCRATCH_BYTES


def domino_attn_block_fwd_workspace_size(desc: AttnDesc) -> int:
    return int(load().domino_attn_block_fwd_workspace_size(ctypes.byref(desc)))


def domino_block_bwd(desc: MlpDesc, X, A_s, B_s, Hpre, H, dY, dHpre, dX_own, peer_dX, dX, dA_s, dB_s,
                     accumulate: int = 0, workspace=None, workspace_bytes: int = 0, compute=None, comm=None,
                     d_b1_s=None):
    _check(load().domino_block_bwd(ctypes.byref(desc), _ptr(X), _ptr(A_s), _ptr(B_s), _ptr(Hpre), _ptr(H), _ptr(dY),
                                   _ptr(dHpre), _ptr(dX_own), _ptr_array(peer_dX), _ptr(dX), _ptr(dA_s), _ptr(dB_s),
                                   _ptr(d_b1_s), int(accumulate), _ptr(workspace), int(workspace_bytes), _stream(compute),
                                   _stream(comm)))


def domino_attn_block_fwd(desc: AttnDesc, X, A_qkv_s, B_o_s, QKV, O, Y_own, peer_Y, Y, workspace=None,
                          workspace_bytes: int = 0, compute=None, comm=None, lse=None, b_qkv_s=None):
    _check(load().domino_attn_block_fwd(ctypes.byref(desc), _ptr(X), _ptr(A_qkv_s), _ptr(B_o_s), _ptr(b_qkv_s),
                                        _ptr(QKV), _ptr(O),
                                        _ptr(lse), _ptr(Y_own), _ptr_array(peer_Y), _ptr(Y), _ptr(workspace),
                                        int(workspace_bytes), _stream(compute), _stream(comm)))


def domino_attn_block_bwd(desc: AttnDesc, X, A_qkv_s, B_o_s, QKV, O, lse, dY, dO, dQKV, dX_own, peer_dX, dX,
                          dA_qkv_s, dB_o_s, accumulate: int = 0, workspace=None, workspace_bytes: int = 0,
                          compute=None, comm=None, d_b_qkv_s=None):
    _check(load().domino_attn_block_bwd(ctypes.byref(desc), _ptr(X), _ptr(A_qkv_s), _ptr(B_o_s), _ptr(QKV), _ptr(O),
                                        _ptr(lse), _ptr(dY), _ptr(dO), _ptr(dQKV), _ptr(dX_own),
                                        _ptr_array(peer_dX), _ptr(dX), _ptr(dA_qkv_s), _ptr(dB_o_s),
                                        _ptr(d_b_qkv_s), int(accumulate), _ptr(workspace), int(workspace_bytes), _stream(compute),
                                        _stream(comm)))


def domino_attn_block_bwd_workspace_size(desc: AttnDesc) -> int:
    return int(load().domino_attn_block_bwd_workspace_size(ctypes.byref(desc)))


def domino_resid_ln_fwd(desc: GroupDesc, resid, y, bias, keep, resid_out, gamma, beta, ln_out, mean, rstd,
                        stream=None):
    _check(load().domino_resid_ln_fwd(ctypes.byref(desc), _ptr(resid), _ptr(y), _ptr(bias), _ptr(keep),
                                      _ptr(resid_out), _ptr(gamma), _ptr(beta), _ptr(ln_out), _ptr(mean), _ptr(rstd),
                                      _stream(stream)))


def domino_resid_ln_bwd(desc: GroupDesc, d_ln, d_res, resid_out, mean, rstd, gamma, keep, d_resid, d_y, d_gamma,
                        d_beta, d_bias, accumulate: int, workspace, workspace_bytes: int, stream=None):
    _check(load().domino_resid_ln_bwd(ctypes.byref(desc), _ptr(d_ln), _ptr(d_res), _ptr(resid_out), _ptr(mean),
                                      _ptr(rstd), _ptr(gamma), _ptr(keep), _ptr(d_resid), _ptr(d_y), _ptr(d_gamma),
                                      _ptr(d_beta), _ptr(d_bias), int(accumulate), _ptr(workspace), workspace_bytes,
                                      _stream(stream)))


def domino_resid_ln_bwd_workspace_size(desc: GroupDesc) -> int:
    return int(load().domino_resid_ln_bwd_workspace_size(ctypes.byref(desc)))


def _struct_of(cls, fields: dict, keep: list):
    """A ctypes struct from a dict of tensors / ints / None (HOST pointer arrays for lists)."""
    st = cls()
    for name, ftype in cls._fields_:
        v = fields.get(name)
        if isinstance(v, (list, tuple)):
            arr = _ptr_array(v)
            keep.append(arr)
            setattr(st, name, ctypes.cast(arr, ftype))
        else:
            setattr(st, name, _ptr(v))
    return st


def domino_stack_fwd(desc: LayerDesc, X, params: Sequence[dict], acts: Sequence[dict], out, workspace=None,
                     workspace_bytes: int = 0, compute=None, comm=None):
    """params / acts: one dict per layer with the fields of domino_layer_params / domino_layer_acts
    (tensors, None, or for peer_y_attn / peer_y_mlp a list of tensors)."""
    keep: list = []
    pa = (LayerParams * len(params))(*[_struct_of(LayerParams, p, keep) for p in params])
    aa = (LayerActs * len(acts))(*[_struct_of(LayerActs, a, keep) for a in acts])
    _check(load().domino_stack_fwd(ctypes.byref(desc), _ptr(X), pa, aa, _ptr(out), _ptr(workspace), workspace_bytes,
                                   _stream(compute), _stream(comm)))


def domino_stack_bwd(desc: LayerDesc, X, params: Sequence[dict], acts: Sequence[dict], grads: Sequence[dict], d_out,
                     dX, accumulate: int, workspace, workspace_bytes: int, compute=None, comm=None):
    keep: list = []
    pa = (LayerParams * len(params))(*[_struct_of(LayerParams, p, keep) for p in params])
    aa = (LayerActs * len(acts))(*[_struct_of(LayerActs, a, keep) for a in acts])
    ga = (LayerGrads * len(grads))(*[_struct_of(LayerGrads, g, keep) for g in grads])
    _check(load().domino_stack_bwd(ctypes.byref(desc), _ptr(X), pa, aa, ga, _ptr(d_out), _ptr(dX), int(accumulate),
                                   _ptr(workspace), workspace_bytes, _stream(compute), _stream(comm)))


def domino_stack_bwd_workspace_size(desc: LayerDesc) -> int:
    return int(load().domino_stack_bwd_workspace_size(ctypes.byref(desc)))


def domino_status_string(status: int) -> str:
    return load().domino_status_string(status).decode()


def domino_timing_enable(enable: bool):
    _check(load().domino_timing_enable(1 if enable else 0))


def domino_timing_read(kind) -> tuple:
    """(launches, total_ms) for a kernel class name or number since timing was enabled."""
    k = KERNEL_KINDS[kind] if isinstance(kind, str) else int(kind)
    n, ms = ctypes.c_int64(), ctypes.c_double()
    _check(load().domino_timing_read(k, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def domino_timing_kernel(kind) -> str:
    """The kernel the most recent timed launch of a kernel class ran ("" if none)."""
    k = KERNEL_KINDS[kind] if isinstance(kind, str) else int(kind)
    buf = ctypes.create_string_buffer(256)
    _check(load().domino_timing_kernel(k, buf, len(buf)))
    return buf.value.decode()
