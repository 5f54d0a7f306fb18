"""ctypes declarations of libbimamba's C ABI (include/bimamba.h)."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbimamba.so")

F32 = 0
BF16 = 1

OK = 0
EINVAL = -1
EUNSUPPORTED = -2
ENOMEM = -3
EHIP = -4
EWORKSPACE = -5

EXPORTS = (
    "bimamba_ssd_workspace_size", "bimamba_ssd_fwd", "bimamba_state_alloc",
    "bimamba_state_reset", "bimamba_state_data", "bimamba_state_free",
    "bimamba_block_step", "bimamba_seq_index", "bimamba_status_str",
    "bimamba_last_error", "bimamba_version", "bimamba_profile_begin",
    "bimamba_profile_end", "bimamba_conv1d_workspace_size", "bimamba_conv1d",
    "bimamba_ssd_bwd_workspace_size", "bimamba_ssd_bwd", "bimamba_gated_norm",
    "bimamba_ssd_fwd_streams", "bimamba_merge_linear", "bimamba_ssd_fwd_noalloc",
    "bimamba_state_alloc_conv", "bimamba_state_conv_ctx", "bimamba_block_step_conv",
)
NOALLOC_SCRATCH_BYTES = 64 << 20


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int), ("seqlen", ctypes.c_int),
                ("nheads", ctypes.c_int), ("headdim", ctypes.c_int),
                ("d_state", ctypes.c_int), ("ngroups", ctypes.c_int),
                ("chunk", ctypes.c_int), ("dtype", ctypes.c_int),
                ("flags", ctypes.c_int)]


class Dir(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("dt", ctypes.c_void_p),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p),
                ("C", ctypes.c_void_p), ("D", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p)]


DT_SOFTPLUS = 1


class Grad(ctypes.Structure):
    _fields_ = [("dx", ctypes.c_void_p), ("ddt", ctypes.c_void_p),
                ("dA", ctypes.c_void_p), ("dB", ctypes.c_void_p),
                ("dC", ctypes.c_void_p), ("dD", ctypes.c_void_p)]


class ConvShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int), ("seqlen", ctypes.c_int),
                ("nheads", ctypes.c_int), ("headdim", ctypes.c_int),
                ("d_state", ctypes.c_int), ("ngroups", ctypes.c_int),
                ("width", ctypes.c_int), ("dtype", ctypes.c_int),
                ("activation", ctypes.c_int), ("flags", ctypes.c_int)]


class ConvDir(ctypes.Structure):
    _fields_ = [("xbc", ctypes.c_void_p), ("weight", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("B", ctypes.c_void_p), ("C", ctypes.c_void_p)]


_LIB = None


class LibraryMissing(RuntimeError):
    pass


def load():
    """Load libbimamba.so; raises LibraryMissing when it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} is not built; run python bidirectional_mamba_ssm_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
    sp, dp = ctypes.POINTER(Shape), ctypes.POINTER(Dir)
    lib.bimamba_ssd_workspace_size.argtypes = [sp, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.bimamba_ssd_fwd.argtypes = [sp, dp, dp, i32p, ctypes.c_int, vp, vp, vp,
                                    vp, ctypes.c_size_t, vp]
    lib.bimamba_state_alloc.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int]
    lib.bimamba_state_reset.argtypes = [vp, i32p, ctypes.c_int, vp]
    lib.bimamba_state_data.argtypes = [vp]
    lib.bimamba_state_data.restype = vp
    lib.bimamba_state_free.argtypes = [vp]
    lib.bimamba_block_step.argtypes = [vp, sp, dp, dp, ctypes.c_int, vp, vp]
    lib.bimamba_seq_index.argtypes = [i32p, ctypes.c_int, ctypes.c_int, vp, vp]
    lib.bimamba_status_str.argtypes = [ctypes.c_int]
    lib.bimamba_status_str.restype = ctypes.c_char_p
    lib.bimamba_last_error.restype = ctypes.c_char_p
    lib.bimamba_version.restype = ctypes.c_int
    lib.bimamba_profile_end.argtypes = [ctypes.c_char_p, ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int),
                                        ctypes.POINTER(ctypes.c_double), ctypes.c_int]
    gp = ctypes.POINTER(Grad)
    lib.bimamba_ssd_bwd_workspace_size.argtypes = [sp, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.bimamba_ssd_bwd.argtypes = [sp, dp, dp, vp, gp, gp, vp, ctypes.c_size_t, vp]
    lib.bimamba_ssd_fwd_streams.argtypes = [sp, dp, dp, i32p, ctypes.c_int, vp, vp, vp, vp,
                                            vp, ctypes.c_size_t, vp]
    lib.bimamba_ssd_fwd_noalloc.argtypes = [sp, dp, dp, i32p, ctypes.c_int, vp, vp, vp, vp]
    lib.bimamba_merge_linear.argtypes = [ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                         vp, vp, vp, vp, vp, vp]
    lib.bimamba_gated_norm.argtypes = [ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       vp, vp, vp, ctypes.c_float, vp, vp]
    csp, cdp = ctypes.POINTER(ConvShape), ctypes.POINTER(ConvDir)
    lib.bimamba_conv1d_workspace_size.argtypes = [csp, ctypes.c_int,
                                                  ctypes.POINTER(ctypes.c_size_t)]
    lib.bimamba_conv1d.argtypes = [csp, cdp, cdp, i32p, ctypes.c_int, vp, vp, vp,
                                   ctypes.c_size_t, vp]
    lib.bimamba_state_alloc_conv.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int]
    lib.bimamba_state_conv_ctx.argtypes = [vp]
    lib.bimamba_state_conv_ctx.restype = vp
    lib.bimamba_block_step_conv.argtypes = [vp, csp, cdp, cdp, sp, dp, dp, ctypes.c_int, vp, vp]
    for name in EXPORTS:
        getattr(lib, name).restype = getattr(lib, name).restype or ctypes.c_int
    _LIB = lib
    return lib


class BimambaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


def check(rc):
    if rc != OK:
        lib = load()
        raise BimambaError(rc, lib.bimamba_last_error().decode(errors="replace"))
