"""ctypes loader for libssm_scan.so (the C ABI declared in include/ssm_scan.h).

The library is built in-tree by ``selective_state_space_38_amd.build``.  There
is no fallback: if the shared library is missing, loading raises.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SSM_SCAN_LIB names another build of the same library (the host-sanitized
# build that the CPU tests run the argument checks against); unset, the in-tree
# library is loaded
LIB_PATH = os.environ.get("SSM_SCAN_LIB") or os.path.join(HERE, "libssm_scan.so")
# the roofline ceiling probes (include/ssm_micro.h), used by the benchmark
MICRO_LIB_PATH = os.path.join(HERE, "libssm_micro.so")
EXPORTED_MICRO = ("ssm_micro_valu", "ssm_micro_stream")

SSM_F32 = 0
SSM_BF16 = 1

SSM_BBAR_DELTA = 0
SSM_BBAR_ZOH = 1

EXPORTED = (
    "selective_scan_fwd",
    "selective_scan_fwd_h0",
    "selective_scan_fwd_noalloc",
    "selective_scan_fwd_ex",
    "selective_scan_fwd_aggregate",
    "selective_scan_carry_combine",
    "ssm_fwd_record_bytes",
    "selective_scan_fwd_aggregate_rec",
    "selective_scan_fwd_from_rec",
    "selective_scan_bwd",
    "selective_scan_fwd_train",
    "selective_scan_bwd_ckpt",
    "selective_scan_fwd_train_ex",
    "selective_scan_bwd_ex",
    "ssm_ckpt_bytes",
    "selective_state_update",
    "selective_state_update_ex",
    "causal_conv1d_fwd",
    "causal_conv1d_update",
    "mamba_block_fwd",
    "ssm_status_string",
    "ssm_check_device_errors",
    "ssm_fwd_plan_for",
)


class SsmDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("dim", ctypes.c_int64),
        ("dstate", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
    ]


class SsmFwdPlan(ctypes.Structure):
    _fields_ = [
        ("state_groups", ctypes.c_int32),
        ("states_per_group", ctypes.c_int32),
        ("segments", ctypes.c_int32),
        ("segment_len", ctypes.c_int32),
        ("lookback", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("workgroups", ctypes.c_int64),
        ("whole_chains", ctypes.c_int32),
        ("first_segment_len", ctypes.c_int32),
        ("helper_waves", ctypes.c_int32),
    ]


class MambaBlockWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("in_x", "in_z", "conv_w", "conv_b", "x_dt", "x_B", "x_C", "dt", "dt_bias",
                 "A", "D", "out")]


class MambaBlockDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("d_model", ctypes.c_int64),
        ("d_inner", ctypes.c_int64),
        ("d_state", ctypes.c_int64),
        ("dt_rank", ctypes.c_int64),
        ("conv_width", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


_lib = None
_micro = None


def load_micro():
    """Returns the loaded probe library, raising if it has not been built."""
    global _micro
    if _micro is not None:
        return _micro
    if not os.path.exists(MICRO_LIB_PATH):
        raise RuntimeError(
            f"{MICRO_LIB_PATH} not found: build it with "
            "`python -m selective_state_space_38_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(MICRO_LIB_PATH)
    vp = ctypes.c_void_p
    lib.ssm_micro_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                   vp, ctypes.c_int, ctypes.POINTER(ctypes.c_float), vp]
    lib.ssm_micro_valu.restype = ctypes.c_int
    lib.ssm_micro_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp,
                                     ctypes.c_int64, ctypes.c_int, vp, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_float), vp]
    lib.ssm_micro_stream.restype = ctypes.c_int
    _micro = lib
    return lib


def load():
    """Returns the loaded library, raising if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} not found: build it with "
            "`python -m selective_state_space_38_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    dims_p = ctypes.POINTER(SsmDims)
    lib.selective_scan_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                       vp, vp, dims_p, vp]
    lib.selective_scan_fwd.restype = ctypes.c_int
    lib.selective_scan_fwd_h0.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                          vp, vp, vp, dims_p, vp]
    lib.selective_scan_fwd_h0.restype = ctypes.c_int
    lib.selective_scan_fwd_noalloc.argtypes = lib.selective_scan_fwd_h0.argtypes
    lib.selective_scan_fwd_noalloc.restype = ctypes.c_int
    lib.selective_scan_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                          vp, ctypes.c_int, vp, vp, dims_p, vp]
    lib.selective_scan_fwd_ex.restype = ctypes.c_int
    lib.selective_scan_fwd_aggregate.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, vp,
                                                 ctypes.c_int, vp, vp, dims_p, vp]
    lib.selective_scan_fwd_aggregate.restype = ctypes.c_int
    lib.selective_scan_carry_combine.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int64,
                                                 dims_p, vp]
    lib.selective_scan_carry_combine.restype = ctypes.c_int
    lib.ssm_fwd_record_bytes.argtypes = [dims_p]
    lib.ssm_fwd_record_bytes.restype = ctypes.c_int64
    lib.selective_scan_fwd_aggregate_rec.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int,
                                                     ctypes.c_int, vp, vp, vp, dims_p, vp]
    lib.selective_scan_fwd_aggregate_rec.restype = ctypes.c_int
    lib.selective_scan_fwd_from_rec.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                                vp, ctypes.c_int, vp, vp, vp, dims_p, vp]
    lib.selective_scan_fwd_from_rec.restype = ctypes.c_int
    lib.selective_scan_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                                       vp, vp, vp, vp, vp, vp, vp, vp, vp, dims_p, vp]
    lib.selective_scan_bwd.restype = ctypes.c_int
    lib.selective_scan_fwd_train.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp,
                                             vp, vp, vp, dims_p, vp]
    lib.selective_scan_fwd_train.restype = ctypes.c_int
    lib.selective_scan_bwd_ckpt.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp,
                                            vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            dims_p, vp]
    lib.selective_scan_bwd_ckpt.restype = ctypes.c_int
    lib.selective_scan_fwd_train_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                                vp, ctypes.c_int, vp, vp, vp, dims_p, vp]
    lib.selective_scan_fwd_train_ex.restype = ctypes.c_int
    lib.selective_scan_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp,
                                          ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          vp, vp, vp, dims_p, vp]
    lib.selective_scan_bwd_ex.restype = ctypes.c_int
    lib.ssm_ckpt_bytes.argtypes = [dims_p]
    lib.ssm_ckpt_bytes.restype = ctypes.c_int64
    lib.selective_state_update.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                           vp, dims_p, vp]
    lib.selective_state_update.restype = ctypes.c_int
    lib.selective_state_update_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              ctypes.c_int, ctypes.c_int, vp, dims_p, vp]
    lib.selective_state_update_ex.restype = ctypes.c_int
    lib.causal_conv1d_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, vp, vp,
                                      dims_p, vp]
    lib.causal_conv1d_fwd.restype = ctypes.c_int
    lib.causal_conv1d_update.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, vp, dims_p,
                                         vp]
    lib.causal_conv1d_update.restype = ctypes.c_int
    lib.mamba_block_fwd.argtypes = [vp, ctypes.POINTER(MambaBlockWeights), vp,
                                    ctypes.POINTER(MambaBlockDims), vp]
    lib.mamba_block_fwd.restype = ctypes.c_int
    lib.ssm_status_string.argtypes = [ctypes.c_int]
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_check_device_errors.argtypes = [vp]
    lib.ssm_check_device_errors.restype = ctypes.c_int
    lib.ssm_fwd_plan_for.argtypes = [dims_p, ctypes.POINTER(SsmFwdPlan)]
    lib.ssm_fwd_plan_for.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(rc):
    return load().ssm_status_string(int(rc)).decode()
