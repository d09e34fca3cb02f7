"""ctypes mirror of include/dmtp.h and the loader of libdmtp.so.

Nothing here computes: it loads the library (failing loudly when it is not
built), mirrors the descriptor structs field for field, and checks at import
that their sizes equal the library's own sizeof values.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_int32, c_size_t, c_uint64, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdmtp.so")

DMTP_F32 = 0
DMTP_BF16 = 1
DMTP_NO_DRAW = 0xFFFFFFFFFFFFFFFF

STATUS = {
    0: "DMTP_OK", -1: "DMTP_E_NULL", -2: "DMTP_E_SHAPE", -3: "DMTP_E_DTYPE",
    -4: "DMTP_E_WORKSPACE", -5: "DMTP_E_ALIGN", -6: "DMTP_E_DEVICE", -7: "DMTP_E_LAUNCH",
    -8: "DMTP_E_ARG", -9: "DMTP_E_SCRATCH",
}


class Rows(ctypes.Structure):
    _fields_ = [("rows", c_void_p), ("dtype", c_int32), ("ids", c_void_p), ("table", c_void_p),
                ("table_rows", c_int32)]


class FuseDesc(ctypes.Structure):
    _fields_ = [("rows", c_int32), ("H", c_int32), ("w_dtype", c_int32), ("eps", c_float),
                ("x1", Rows), ("x2", Rows), ("res", Rows), ("g1", c_void_p), ("g2", c_void_p),
                ("W", c_void_p), ("out", c_void_p)]


class Layer(ctypes.Structure):
    _fields_ = [("g_attn", c_void_p), ("wqkv", c_void_p), ("wo", c_void_p), ("g_ffn", c_void_p),
                ("wg", c_void_p), ("wu", c_void_p), ("wd", c_void_p), ("ctx_k", c_void_p),
                ("ctx_v", c_void_p)]


class DraftDesc(ctypes.Structure):
    _fields_ = [("B", c_int32), ("H", c_int32), ("Hq", c_int32), ("Hkv", c_int32), ("d", c_int32),
                ("F", c_int32), ("n_layers", c_int32), ("K", c_int32), ("n_anchor", c_int32),
                ("dtype", c_int32), ("eps", c_float), ("rope_base", c_float), ("window", c_int32),
                ("max_ctx", c_int32), ("ctx_rows", c_int32), ("V", c_int32),
                ("anchor_ids", c_void_p), ("x_t1", c_void_p), ("mask_id", c_int32),
                ("emb", c_void_p), ("cu_ctx", c_void_p), ("layers", POINTER(Layer)),
                ("g_final", c_void_p), ("out", c_void_p),
                ("attn_start_event", c_void_p), ("attn_stop_event", c_void_p)]


class HeadSegment(ctypes.Structure):
    _fields_ = [("x", c_void_p), ("n", c_int32), ("ld", c_int32), ("dtype", c_int32),
                ("g_norm", c_void_p)]


class HeadDesc(ctypes.Structure):
    _fields_ = [("H", c_int32), ("V", c_int32), ("dtype", c_int32), ("eps", c_float),
                ("n_seg", c_int32), ("seg", HeadSegment * 4), ("W", c_void_p),
                ("temperature", c_void_p), ("draw_key", c_void_p), ("seed", c_uint64),
                ("plant_row", c_void_p), ("store_row", c_void_p), ("logits", c_void_p),
                ("logits_rows", c_int32), ("prepared", c_void_p), ("token", c_void_p),
                ("row_max", c_void_p), ("lse", c_void_p), ("gap", c_void_p),
                ("gemm_start_event", c_void_p), ("gemm_stop_event", c_void_p),
                ("w_packed", c_void_p)]


class VerifyDesc(ctypes.Structure):
    _fields_ = [("B", c_int32), ("K", c_int32), ("V", c_int32), ("t1", c_void_p),
                ("drafts", c_void_p), ("target", c_void_p), ("temperature", c_void_p),
                ("logits", c_void_p), ("t1_lse", c_void_p), ("draft_lse", c_void_p),
                ("target_lse", c_void_p), ("u_acc", c_void_p), ("seed", c_uint64),
                ("final_key", c_void_p), ("accept_len", c_void_p), ("out_tokens", c_void_p),
                ("n_out", c_void_p), ("target_only", c_int32),
                ("mass_start_event", c_void_p), ("mass_stop_event", c_void_p)]


class StatsDesc(ctypes.Structure):
    _fields_ = [("B", c_int32), ("K", c_int32), ("accept_len", c_void_p), ("hist", c_void_p),
                ("summary", c_void_p)]


class MtpDesc(ctypes.Structure):
    _fields_ = [("B", c_int32), ("S", c_int32), ("H", c_int32), ("Hq", c_int32), ("Hkv", c_int32),
                ("d", c_int32), ("F", c_int32), ("n_layers", c_int32), ("dtype", c_int32),
                ("eps", c_float), ("rope_base", c_float), ("max_ctx", c_int32),
                ("ctx_rows", c_int32), ("x", c_void_p), ("cu_ctx", c_void_p),
                ("layers", POINTER(Layer)), ("out", c_void_p), ("k_new", POINTER(c_void_p)),
                ("v_new", POINTER(c_void_p))]


class CtxDesc(ctypes.Structure):
    _fields_ = [("N", c_int32), ("n_feat", c_int32), ("H", c_int32), ("Hq", c_int32),
                ("Hkv", c_int32), ("d", c_int32), ("n_layers", c_int32), ("dtype", c_int32),
                ("eps", c_float), ("rope_base", c_float), ("feats", c_void_p),
                ("positions", c_void_p), ("dst_rows", c_void_p), ("w_fc", c_void_p),
                ("layers", POINTER(Layer)), ("ctx_rows", c_int32), ("k_cache", POINTER(c_void_p)),
                ("v_cache", POINTER(c_void_p)), ("ctx_out", c_void_p)]


_STRUCTS = [Rows, FuseDesc, Layer, DraftDesc, HeadSegment, HeadDesc, VerifyDesc, StatsDesc,
            MtpDesc, CtxDesc]

# exported symbols of include/dmtp.h
SYMBOLS = ["dmtp_fuse", "dmtp_fuse_ws", "dmtp_fuse_noalloc", "dmtp_mtp_block", "dmtp_mtp_block_ws", "dmtp_ctx_kv",
           "dmtp_ctx_kv_ws", "dmtp_block_draft",
           "dmtp_block_draft_ws", "dmtp_lm_head",
           "dmtp_lm_head_ws", "dmtp_head_pack", "dmtp_head_pack_bytes", "dmtp_verify", "dmtp_verify_ws", "dmtp_accept_stats",
           "dmtp_status_str", "dmtp_version", "dmtp_struct_size"]


class DmtpError(RuntimeError):
    def __init__(self, call: str, status: int, msg: str):
        super().__init__(f"{call} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m mtp_block_draft_amd.build` "
                          "(the DMTP path has no fallback)")
    lib = ctypes.CDLL(path)
    for name, desc in (("dmtp_fuse", FuseDesc), ("dmtp_mtp_block", MtpDesc), ("dmtp_ctx_kv", CtxDesc),
                       ("dmtp_block_draft", DraftDesc),
                       ("dmtp_lm_head", HeadDesc), ("dmtp_verify", VerifyDesc)):
        f = getattr(lib, name)
        f.argtypes = [POINTER(desc), c_void_p, c_size_t, c_void_p]
        f.restype = c_int
        q = getattr(lib, name + "_ws")
        q.argtypes = [POINTER(desc)]
        q.restype = c_size_t
    lib.dmtp_fuse_noalloc.argtypes = [POINTER(FuseDesc), c_void_p]
    lib.dmtp_fuse_noalloc.restype = c_int
    lib.dmtp_head_pack_bytes.argtypes = [c_int32, c_int32]
    lib.dmtp_head_pack_bytes.restype = c_size_t
    lib.dmtp_head_pack.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_size_t, c_void_p]
    lib.dmtp_head_pack.restype = c_int
    lib.dmtp_accept_stats.argtypes = [POINTER(StatsDesc), c_void_p]
    lib.dmtp_accept_stats.restype = c_int
    lib.dmtp_status_str.argtypes = [c_int]
    lib.dmtp_status_str.restype = ctypes.c_char_p
    lib.dmtp_version.argtypes = []
    lib.dmtp_version.restype = ctypes.c_char_p
    lib.dmtp_struct_size.argtypes = [c_int]
    lib.dmtp_struct_size.restype = c_size_t
    for i, st in enumerate(_STRUCTS):
        n = lib.dmtp_struct_size(i)
        if n != ctypes.sizeof(st):
            raise ImportError(f"ABI mismatch: {st.__name__} is {ctypes.sizeof(st)} bytes here, "
                              f"{n} in the library")
    return lib
