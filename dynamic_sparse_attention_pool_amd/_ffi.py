"""ctypes mirror of include/sa.h and loader for libsa.so.

Only argument marshalling lives here: every step of the path runs in the HIP
kernels of libsa.so.  Loading fails loudly when the library has not been
built (there is no fallback).
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsa.so")

SA_OK = 0
SA_F32, SA_BF16, SA_I32 = 0, 1, 2
SA_EST_BLOCK_MEANPOOL, SA_EST_VSLASH, SA_EST_CENTROID, SA_EST_INDEXER = 0, 1, 2, 3
SA_FWD_BLOCK, SA_FWD_VSLASH, SA_FWD_ASHAPE = 0, 1, 2
SA_GATHER_CLUSTER, SA_GATHER_TOKEN = 0, 1
ABI_VERSION = 9
STATIC_SCRATCH_BYTES = 32 << 20   # SA_STATIC_SCRATCH_BYTES

STATUS_NAMES = {0: "SA_OK", 1: "SA_ERR_NULL", 2: "SA_ERR_SHAPE", 3: "SA_ERR_DTYPE", 4: "SA_ERR_ALIGN",
                5: "SA_ERR_WORKSPACE", 6: "SA_ERR_UNSUPPORTED", 7: "SA_ERR_LAUNCH", 8: "SA_ERR_VALUE"}

P = C.c_void_p
I32P = C.POINTER(C.c_int32)
F32P = C.POINTER(C.c_float)


class EstimateArgs(C.Structure):
    _fields_ = [("kind", C.c_int32), ("dtype", C.c_int32), ("batch", C.c_int64), ("heads_q", C.c_int64),
                ("heads_kv", C.c_int64), ("seq_q", C.c_int64), ("seq_k", C.c_int64), ("head_dim", C.c_int64),
                ("n_centroids", C.c_int64), ("q_pos0", C.c_int64), ("block_size", C.c_int32),
                ("last_q", C.c_int32), ("scale", C.c_float), ("reserved0", C.c_int32), ("q", P), ("k", P),
                ("centroids", P), ("weights", P), ("scores", P), ("scores2", P), ("pooled_q", P),
                ("pooled_k", P), ("head_list", P), ("n_heads_list", C.c_int32), ("reserved1", C.c_int32),
                ("err_flag", P)]


class SelectArgs(C.Structure):
    _fields_ = [("scores", P), ("rows", C.c_int64), ("ncand", C.c_int64), ("ld", C.c_int64),
                ("causal_period", C.c_int64), ("causal_offset", C.c_int64), ("causal", C.c_int32),
                ("n_sink", C.c_int32), ("n_local", C.c_int32), ("k", C.c_int32), ("ratio_num", C.c_int32),
                ("ratio_den", C.c_int32), ("kmax", C.c_int32), ("reserved0", C.c_int32), ("idx", P),
                ("cnt", P), ("err_flag", P)]


class VsBuildArgs(C.Structure):
    _fields_ = [("rows", C.c_int64), ("seq", C.c_int64), ("block_size", C.c_int32), ("n_vert", C.c_int32),
                ("n_slash", C.c_int32), ("reserved0", C.c_int32), ("vert", P), ("vert_cnt", P), ("slash", P),
                ("slash_cnt", P), ("iv", P), ("iv_cnt", P), ("col", P), ("col_cnt", P)]


class FwdArgs(C.Structure):
    _fields_ = [("mode", C.c_int32), ("dtype", C.c_int32), ("out_dtype", C.c_int32), ("block_size", C.c_int32),
                ("batch", C.c_int64), ("heads_q", C.c_int64), ("heads_kv", C.c_int64), ("seq", C.c_int64),
                ("head_dim", C.c_int64), ("scale", C.c_float), ("kmax", C.c_int32), ("q", P), ("k", P),
                ("v", P), ("out", P), ("lse", P), ("block_idx", P), ("block_cnt", P), ("iv", P),
                ("iv_cnt", P), ("col", P), ("col_cnt", P), ("max_iv", C.c_int32), ("max_col", C.c_int32),
                ("n_sink", C.c_int32), ("n_local", C.c_int32), ("head_list", P), ("n_heads_list", C.c_int32),
                ("reserved1", C.c_int32)]


class GatherArgs(C.Structure):
    _fields_ = [("mode", C.c_int32), ("dtype", C.c_int32), ("out_dtype", C.c_int32), ("n_clusters", C.c_int32),
                ("n_q", C.c_int64), ("heads_q", C.c_int64), ("heads_kv", C.c_int64), ("n_ctx", C.c_int64),
                ("head_dim", C.c_int64), ("scale", C.c_float), ("n_sel", C.c_int32), ("n_tok", C.c_int32),
                ("tok_per_head", C.c_int32), ("q", P), ("k", P), ("v", P), ("cluster_ptr", P), ("sel", P),
                ("tok_idx", P), ("out", P), ("lse", P), ("q_pos", P), ("perm", P)]


class ClusterPackArgs(C.Structure):
    _fields_ = [("heads_kv", C.c_int64), ("n_ctx", C.c_int64), ("head_dim", C.c_int64),
                ("n_clusters", C.c_int32), ("dtype", C.c_int32), ("labels", P), ("cluster_ptr", P),
                ("perm", P), ("k", P), ("v", P), ("k_packed", P), ("v_packed", P), ("err_flag", P)]


class SelectMassArgs(C.Structure):
    _fields_ = [("scores", P), ("rows", C.c_int64), ("ncand", C.c_int64), ("ld", C.c_int64),
                ("mass", C.c_float), ("k_min", C.c_int32), ("k_max", C.c_int32), ("kmax", C.c_int32),
                ("idx", P), ("cnt", P), ("err_flag", P)]


class KmeansArgs(C.Structure):
    _fields_ = [("heads_kv", C.c_int64), ("n_ctx", C.c_int64), ("head_dim", C.c_int64), ("n_clusters", C.c_int32),
                ("iters", C.c_int32), ("dtype", C.c_int32), ("reserved0", C.c_int32), ("k", P), ("centroids", P),
                ("labels", P), ("cluster_ptr", P), ("perm", P)]


class EstimateTopkArgs(C.Structure):
    _fields_ = [("kind", C.c_int32), ("dtype", C.c_int32), ("batch", C.c_int64), ("heads_q", C.c_int64),
                ("heads_kv", C.c_int64), ("seq", C.c_int64), ("head_dim", C.c_int64), ("block_size", C.c_int32),
                ("scale", C.c_float), ("n_sink", C.c_int32), ("n_local", C.c_int32), ("k", C.c_int32),
                ("ratio_num", C.c_int32), ("ratio_den", C.c_int32), ("kmax", C.c_int32), ("q", P), ("k_ptr", P),
                ("pooled_q", P), ("pooled_k", P), ("head_list", P), ("n_heads_list", C.c_int32),
                ("n_centroids", C.c_int32), ("idx", P), ("cnt", P), ("err_flag", P), ("mass", C.c_float),
                ("k_min", C.c_int32)]


class IndexerTopkArgs(C.Structure):
    _fields_ = [("seq_q", C.c_int64), ("seq_k", C.c_int64), ("q_pos0", C.c_int64), ("heads", C.c_int32),
                ("head_dim", C.c_int32), ("k", C.c_int32), ("kmax", C.c_int32), ("q", P), ("k_ptr", P),
                ("weights", P), ("idx", P), ("cnt", P), ("err_flag", P)]


STRUCTS = [EstimateArgs, SelectArgs, VsBuildArgs, FwdArgs, GatherArgs, ClusterPackArgs, SelectMassArgs, KmeansArgs,
           EstimateTopkArgs, IndexerTopkArgs]

# exported symbol -> (restype, argtypes)
SYMBOLS = {
    "sa_estimate": (C.c_int, [C.POINTER(EstimateArgs), P, C.c_size_t, P]),
    "sa_estimate_workspace_bytes": (C.c_int, [C.POINTER(EstimateArgs), C.POINTER(C.c_size_t)]),
    "sa_select_topk": (C.c_int, [C.POINTER(SelectArgs), P, C.c_size_t, P]),
    "sa_select_topk_workspace_bytes": (C.c_int, [C.POINTER(SelectArgs), C.POINTER(C.c_size_t)]),
    "sa_select_mass": (C.c_int, [C.POINTER(SelectMassArgs), P]),
    "sa_vs_build": (C.c_int, [C.POINTER(VsBuildArgs), P]),
    "sa_block_sparse_fwd": (C.c_int, [C.POINTER(FwdArgs), P, C.c_size_t, P]),
    "sa_block_sparse_fwd_workspace_bytes": (C.c_int, [C.POINTER(FwdArgs), C.POINTER(C.c_size_t)]),
    "sa_gather_decode": (C.c_int, [C.POINTER(GatherArgs), P, C.c_size_t, P]),
    "sa_gather_decode_workspace_bytes": (C.c_int, [C.POINTER(GatherArgs), C.POINTER(C.c_size_t)]),
    "sa_gather_decode_static": (C.c_int, [C.POINTER(GatherArgs), P]),
    "sa_cluster_pack": (C.c_int, [C.POINTER(ClusterPackArgs), P, C.c_size_t, P]),
    "sa_cluster_pack_workspace_bytes": (C.c_int, [C.POINTER(ClusterPackArgs), C.POINTER(C.c_size_t)]),
    "sa_kmeans": (C.c_int, [C.POINTER(KmeansArgs), P, C.c_size_t, P]),
    "sa_estimate_topk": (C.c_int, [C.POINTER(EstimateTopkArgs), P, C.c_size_t, P]),
    "sa_estimate_topk_workspace_bytes": (C.c_int, [C.POINTER(EstimateTopkArgs), C.POINTER(C.c_size_t)]),
    "sa_kmeans_workspace_bytes": (C.c_int, [C.POINTER(KmeansArgs), C.POINTER(C.c_size_t)]),
    "sa_indexer_topk": (C.c_int, [C.POINTER(IndexerTopkArgs), P, C.c_size_t, P]),
    "sa_indexer_topk_workspace_bytes": (C.c_int, [C.POINTER(IndexerTopkArgs), C.POINTER(C.c_size_t)]),
    "sa_peak_mfma_bf16": (C.c_int, [P, C.c_int, C.c_int, C.POINTER(C.c_double), P]),
    "sa_peak_read": (C.c_int, [P, C.c_size_t, C.c_int, P, C.POINTER(C.c_double), P]),
    "sa_last_error": (C.c_char_p, []),
    "sa_version": (C.c_int, []),
    "sa_args_size": (C.c_size_t, [C.c_int]),
}


class SAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load():
    """Load libsa.so once; raise if it is missing or its ABI does not match."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libsa.so not built at {LIB_PATH}; run __graft_entry__.build() first "
                          "(there is no CPU fallback)")
    # torch's HIP runtime must be the one libsa binds to (same device memory,
    # same streams): loading torch first makes the dynamic loader resolve
    # libsa's libamdhip64 dependency to the copy torch already holds.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SYMBOLS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.sa_version() != ABI_VERSION:
        raise ImportError(f"libsa ABI version {lib.sa_version()} != {ABI_VERSION}")
    for i, st in enumerate(STRUCTS):
        if lib.sa_args_size(i) != C.sizeof(st):
            raise ImportError(f"struct {st.__name__}: library size {lib.sa_args_size(i)} != binding {C.sizeof(st)}")
    _lib = lib
    return lib


def check(rc: int):
    if rc != SA_OK:
        raise SAError(rc, _lib.sa_last_error().decode())
