"""ctypes view of libmpa.so (include/mpa.h).  Loading fails loudly when the
library has not been built: there is no fallback path."""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MPA_LIBRARY names another build of the same library (e.g. to compare builds);
# by default the in-tree one.
LIB_PATH = os.environ.get("MPA_LIBRARY") or os.path.join(_HERE, "lib", "libmpa.so")

c_i32p = ctypes.POINTER(ctypes.c_int32)
c_i64p = ctypes.POINTER(ctypes.c_int64)
c_u64p = ctypes.POINTER(ctypes.c_uint64)
c_vp = ctypes.c_void_p
c_opp = ctypes.POINTER(ctypes.c_void_p)

# name -> (restype, argtypes), in the order of include/mpa.h
SIGNATURES = {
    "mpaSelfAttentionPrefixEncoderGetWorkspaceSize": (ctypes.c_int32, [
        c_vp, c_vp, c_vp, c_vp,                      # query, key, value, blockTables
        c_i32p, c_i32p, c_vp, ctypes.c_int,          # seqLen, kvSeqLen, slopes, maskType
        ctypes.c_int32, ctypes.c_int32, ctypes.c_float,  # headNum, kvHeadNum, qkScale
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,  # batch, headSize, numBlocks, blockSize, maxBlockNum
        ctypes.c_int, c_i64p, ctypes.c_int64,        # dtype, qStartLoc, nTokens
        c_vp, c_vp, c_u64p, c_opp]),                 # attnOut, lse, workspaceSize, op
    "mpaSelfAttentionPrefixEncoderChunkedGetWorkspaceSize": (ctypes.c_int32, [
        c_vp, c_vp, c_vp, c_vp,                      # query, key, value, blockTables
        c_i32p, c_i32p, ctypes.c_int32,              # seqLen, kvSeqLen, attentionChunkSize
        ctypes.c_int32, ctypes.c_int32, ctypes.c_float,  # headNum, kvHeadNum, qkScale
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,  # batch, headSize, numBlocks, blockSize, maxBlockNum
        ctypes.c_int, c_i64p, ctypes.c_int64,        # dtype, qStartLoc, nTokens
        c_vp, c_vp, c_u64p, c_opp]),                 # attnOut, lse, workspaceSize, op
    "mpaSelfAttentionPrefixEncoderCompressedMaskGetWorkspaceSize": (ctypes.c_int32, [
        c_vp, c_vp, c_vp, c_vp,                      # query, key, value, blockTables
        c_i32p, c_i32p,                              # seqLen, kvSeqLen
        c_vp, ctypes.c_int32, ctypes.c_int32,        # mask, maskRows, maskCols
        c_vp, ctypes.c_int,                          # slopes, maskType
        ctypes.c_int32, ctypes.c_int32, ctypes.c_float,  # headNum, kvHeadNum, qkScale
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,  # batch, headSize, numBlocks, blockSize, maxBlockNum
        ctypes.c_int, c_i64p, ctypes.c_int64,        # dtype, qStartLoc, nTokens
        c_vp, c_vp, c_u64p, c_opp]),                 # attnOut, lse, workspaceSize, op
    "mpaSelfAttentionPrefixEncoder": (ctypes.c_int32, [c_vp, ctypes.c_uint64, c_vp, c_vp]),
    "mpaMLAGetWorkspaceSize": (ctypes.c_int32, [
        c_vp, c_vp, c_vp, c_vp, c_vp,                # qNope, qRope, ctKV, kRope, blockTables
        c_i32p, c_i32p,                              # contextLens, qSeqLen
        ctypes.c_int32, ctypes.c_float, ctypes.c_int32,  # headNum, qkScale, kvHeadNum
        ctypes.c_int, ctypes.c_int, ctypes.c_int,    # maskType, calcType, cacheMode
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,  # batch, numBlocks, blockSize, maxBlockNum
        ctypes.c_int, ctypes.c_int64,                # dtype, nTokens
        c_vp, c_vp, c_u64p, c_opp]),                 # attenOut, lse, workspaceSize, op
    "mpaMLAInt8GetWorkspaceSize": (ctypes.c_int32, [
        c_vp, c_vp, c_vp, c_vp, c_vp,                # qNope, qRope, ctKV, kRope, blockTables
        c_i32p, c_i32p, c_vp, c_vp,                  # contextLens, qSeqLen, qkDescale, pvDescale
        ctypes.c_int32, ctypes.c_float, ctypes.c_int32,  # headNum, qkScale, kvHeadNum
        ctypes.c_int, ctypes.c_int,                  # maskType, calcType
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,  # batch, numBlocks, blockSize, maxBlockNum
        ctypes.c_int, ctypes.c_int64,                # dtype, nTokens
        c_vp, c_vp, c_u64p, c_opp]),                 # attenOut, lse, workspaceSize, op
    "mpaMLA": (ctypes.c_int32, [c_vp, ctypes.c_uint64, c_vp, c_vp]),
    "mpaMLAStaticScratch": (ctypes.c_int32, [c_vp, c_vp]),
    "mpaLseMerge": (ctypes.c_int32, [
        c_vp, c_vp, ctypes.c_int32, ctypes.c_int64,  # oParts, lseParts, nParts, rows
        ctypes.c_int32, ctypes.c_int, c_vp, c_vp, c_vp]),  # headDim, dtype, out, lse, stream
    "mpaOperationSetLaunchEvents": (ctypes.c_int32, [c_vp, c_vp, c_vp]),
    "mpaDestroyOperation": (ctypes.c_int32, [c_vp]),
    "mpaGetErrorString": (ctypes.c_char_p, [ctypes.c_int32]),
    "mpaGetLastErrorMessage": (ctypes.c_char_p, []),
    "mpaPrefixEncoderPlanInspect": (ctypes.c_int32, [
        c_i32p, c_i32p, ctypes.c_int32, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, c_i32p, ctypes.c_int64, c_i64p, c_i32p, c_i32p, c_i32p, c_u64p]),
    "mpaMLAPlanInspect": (ctypes.c_int32, [
        c_i32p, c_i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int, c_i32p, ctypes.c_int64,
        c_i64p]),
}


def load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -m masked_paged_attention_amd.build "
            "or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = load()
