"""Masked attention over a paged KV cache on MI355X (gfx950).

Python binding of libmpa.so (C ABI in include/mpa.h).  This module only
marshals arguments -- torch tensors to device pointers, host length arrays to
int32/int64 buffers, the current HIP stream -- and calls the library; every step
of the computation runs in the library's HIP kernels.  Importing fails if the
library is not built.

    import masked_paged_attention_amd as mpa
    out, lse = mpa.prefix_encoder(q, k_cache, v_cache, block_tables, seq_len, kv_seq_len,
                                  mask_type=mpa.MASK_CAUSAL, qk_scale=0.125, return_lse=True)
    out = mpa.mla(q_nope, q_rope, ct_kv, k_rope, block_tables, context_lens, qk_scale=s)

For repeated calls with the same shapes build the operation once
(``PrefixEncoder(...)`` / ``MLA(...)``) and call ``run()``.
"""

import ctypes

import numpy as np
import torch

from ._lib import LIB

MASK_NONE = 0
MASK_ALIBI = 3            # MPA_MASK_ALIBI_COMPRESS
MASK_ALIBI_SQRT = 4       # MPA_MASK_ALIBI_COMPRESS_SQRT
MASK_ALIBI_LEFT = 5       # MPA_MASK_ALIBI_COMPRESS_LEFT_ALIGN
MASK_CAUSAL = 9           # MPA_MASK_CAUSAL
MLA_MASK_UNDEFINED = 0
MLA_MASK_SPEC = 1
MLA_CALC_UNDEFINED = 0
MLA_CALC_SPEC = 1
MLA_CALC_PREFILL = 3
MLA_CACHE_KVCACHE = 0
MLA_CACHE_KROPE_CTKV = 1

MPA_OK = 0
_DTYPES = {torch.float16: 0, torch.bfloat16: 1}


class MpaError(RuntimeError):
    def __init__(self, status, where):
        msg = LIB.mpaGetLastErrorMessage().decode()
        name = LIB.mpaGetErrorString(status).decode()
        super().__init__(f"{where}: {name} ({status}): {msg}")
        self.status = status


def _check(status, where):
    if status != MPA_OK:
        raise MpaError(status, where)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _host_i32(x):
    a = np.ascontiguousarray(np.asarray(x.cpu() if torch.is_tensor(x) else x, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _host_i64(x):
    a = np.ascontiguousarray(np.asarray(x.cpu() if torch.is_tensor(x) else x, dtype=np.int64))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _event(ev):
    if ev is None:
        return ctypes.c_void_p(0)
    handle = ev.cuda_event if hasattr(ev, "cuda_event") else int(ev)
    _need(handle != 0, "the event has no HIP event yet: record it once before attaching it")
    return ctypes.c_void_p(handle)


def _set_launch_events(op, start, stop):
    _check(LIB.mpaOperationSetLaunchEvents(op, _event(start), _event(stop)), "mpaOperationSetLaunchEvents")


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


class PrefixEncoder:
    """A planned PrefixEncoder call (phase 1 of the C ABI); ``run()`` launches it."""

    def __init__(self, query, key, value, block_tables, seq_len, kv_seq_len, *, mask_type,
                 qk_scale, slopes=None, q_start_loc=None, head_num=None, kv_head_num=None,
                 out=None, lse=None, return_lse=False, attention_chunk=None, compressed_mask=None):
        """attention_chunk: chunk size of the chunked local causal mask (then
        mask_type must be MASK_CAUSAL and slopes None).  compressed_mask: an
        explicit compressed mask tile on the device, query's dtype ([128, 128]
        for MASK_CAUSAL, [256, 256] for the ALiBi types), read by the kernel in
        place of the generated mask."""
        _need(query.is_cuda and key.is_cuda and value.is_cuda and block_tables.is_cuda,
              "query, key, value and block_tables must be device tensors")
        _need(query.dtype in _DTYPES and key.dtype == query.dtype and value.dtype == query.dtype,
              "query/key/value must share one dtype, float16 or bfloat16")
        _need(query.dim() == 3 and key.dim() == 4 and value.shape == key.shape,
              "query [nTokens, headNum, headSize]; key/value [numBlocks, blockSize, kvHeadNum, headSize]")
        _need(all(t.is_contiguous() for t in (query, key, value, block_tables)),
              "tensors must be contiguous")
        _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2,
              "block_tables must be int32 [batch, maxBlockNum]")
        n_tokens, H, D = query.shape
        nb, bs, kvh, dk = key.shape
        _need(dk == D, "key/value headSize must equal query headSize")
        _need(head_num in (None, H) and kv_head_num in (None, kvh), "head counts disagree with shapes")
        self._seq, p_seq = _host_i32(seq_len)
        self._kv, p_kv = _host_i32(kv_seq_len)
        B = len(self._seq)
        _need(len(self._kv) == B and block_tables.shape[0] == B, "batch sizes disagree")
        if q_start_loc is not None:
            self._qs, p_qs = _host_i64(q_start_loc)
            _need(len(self._qs) == B, "q_start_loc needs one entry per sequence")
        else:
            self._qs, p_qs = None, ctypes.POINTER(ctypes.c_int64)()
        if slopes is not None:
            if not torch.is_tensor(slopes):
                slopes = torch.as_tensor(np.asarray(slopes, dtype=np.float32), device=query.device)
            _need(slopes.is_cuda and slopes.dtype == torch.float32 and slopes.numel() == H,
                  "slopes must be a float32 device tensor [headNum]")
            slopes = slopes.contiguous()
        self.slopes = slopes
        self.out = out if out is not None else torch.empty_like(query)
        _need(self.out.shape == query.shape and self.out.dtype == query.dtype and self.out.is_contiguous(),
              "out must match query")
        if lse is None and return_lse:
            lse = torch.empty((n_tokens, H), dtype=torch.float32, device=query.device)
        if lse is not None:
            _need(lse.dtype == torch.float32 and tuple(lse.shape) == (n_tokens, H) and lse.is_contiguous(),
                  "lse must be float32 [nTokens, headNum]")
        self.lse = lse
        self._keep = (query, key, value, block_tables)
        self.device = query.device
        ws = ctypes.c_uint64(0)
        op = ctypes.c_void_p(0)
        if compressed_mask is not None:
            _need(attention_chunk is None, "a compressed mask does not combine with attention_chunk")
            _need(compressed_mask.is_cuda and compressed_mask.dtype == query.dtype
                  and compressed_mask.dim() == 2 and compressed_mask.is_contiguous(),
                  "compressed_mask must be a contiguous 2-D device tensor of query's dtype")
            self._keep = self._keep + (compressed_mask,)
            st = LIB.mpaSelfAttentionPrefixEncoderCompressedMaskGetWorkspaceSize(
                _ptr(query), _ptr(key), _ptr(value), _ptr(block_tables), p_seq, p_kv,
                _ptr(compressed_mask), compressed_mask.shape[0], compressed_mask.shape[1], _ptr(slopes),
                int(mask_type), H, kvh, float(qk_scale), B, D, nb, bs, block_tables.shape[1],
                _DTYPES[query.dtype], p_qs, n_tokens, _ptr(self.out), _ptr(lse),
                ctypes.byref(ws), ctypes.byref(op))
            _check(st, "mpaSelfAttentionPrefixEncoderCompressedMaskGetWorkspaceSize")
        elif attention_chunk is None:
            st = LIB.mpaSelfAttentionPrefixEncoderGetWorkspaceSize(
                _ptr(query), _ptr(key), _ptr(value), _ptr(block_tables), p_seq, p_kv, _ptr(slopes),
                int(mask_type), H, kvh, float(qk_scale), B, D, nb, bs, block_tables.shape[1],
                _DTYPES[query.dtype], p_qs, n_tokens, _ptr(self.out), _ptr(lse),
                ctypes.byref(ws), ctypes.byref(op))
            _check(st, "mpaSelfAttentionPrefixEncoderGetWorkspaceSize")
        else:
            _need(int(mask_type) == MASK_CAUSAL and slopes is None,
                  "the chunked local mask is causal and takes no slopes")
            st = LIB.mpaSelfAttentionPrefixEncoderChunkedGetWorkspaceSize(
                _ptr(query), _ptr(key), _ptr(value), _ptr(block_tables), p_seq, p_kv, int(attention_chunk),
                H, kvh, float(qk_scale), B, D, nb, bs, block_tables.shape[1],
                _DTYPES[query.dtype], p_qs, n_tokens, _ptr(self.out), _ptr(lse),
                ctypes.byref(ws), ctypes.byref(op))
            _check(st, "mpaSelfAttentionPrefixEncoderChunkedGetWorkspaceSize")
        self._op = op
        self.workspace = (torch.empty(ws.value, dtype=torch.uint8, device=query.device)
                          if ws.value else None)

    def run(self, stream=None):
        ws = self.workspace
        st = LIB.mpaSelfAttentionPrefixEncoder(_ptr(ws), ws.numel() if ws is not None else 0,
                                               self._op, _stream(self.device, stream))
        _check(st, "mpaSelfAttentionPrefixEncoder")
        return (self.out, self.lse) if self.lse is not None else self.out

    def set_launch_events(self, start=None, stop=None):
        """Later runs record ``start`` / ``stop`` (torch.cuda.Event with timing, already
        created by one record, or None) at their kernel's start and end."""
        _set_launch_events(self._op, start, stop)

    def close(self):
        if getattr(self, "_op", None) is not None and self._op.value:
            LIB.mpaDestroyOperation(self._op)
            self._op = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def prefix_encoder(query, key, value, block_tables, seq_len, kv_seq_len, *,
                   mask_type=MASK_CAUSAL, qk_scale=None, slopes=None, q_start_loc=None,
                   out=None, lse=None, return_lse=False, stream=None, attention_chunk=None,
                   compressed_mask=None):
    """One masked paged-attention call; returns out, or (out, lse) with return_lse."""
    if qk_scale is None:
        qk_scale = 1.0 / float(query.shape[-1]) ** 0.5
    op = PrefixEncoder(query, key, value, block_tables, seq_len, kv_seq_len, mask_type=mask_type,
                       qk_scale=qk_scale, slopes=slopes, q_start_loc=q_start_loc, out=out, lse=lse,
                       return_lse=return_lse, attention_chunk=attention_chunk,
                       compressed_mask=compressed_mask)
    try:
        return op.run(stream)
    finally:
        # Execution is asynchronous; the operation's plan must outlive it.
        torch.cuda.current_stream(query.device).synchronize() if stream is None else stream.synchronize()
        op.close()


class MLA:
    """A planned MLA decode call (phase 1 of the C ABI); ``run()`` launches it.

    With int8 ``q_nope`` and ``ct_kv`` (the int8 latent cache) ``qk_descale`` and
    ``pv_descale`` (float32 [headNum] device tensors) and ``k_rope`` are required;
    q_rope, k_rope and the output then carry the float16/bfloat16 type."""

    def __init__(self, q_nope, q_rope, ct_kv, k_rope, block_tables, context_lens, *, qk_scale,
                 q_seq_len=None, mask_type=MLA_MASK_UNDEFINED, calc_type=None, cache_mode=None,
                 out=None, lse=None, return_lse=False, qk_descale=None, pv_descale=None):
        _need(q_nope.is_cuda and q_rope.is_cuda and ct_kv.is_cuda and block_tables.is_cuda,
              "inputs must be device tensors")
        quant = q_nope.dtype == torch.int8
        dt = q_rope.dtype
        if quant:
            _need(ct_kv.dtype == torch.int8 and k_rope is not None and k_rope.dtype == dt and dt in _DTYPES,
                  "int8 cache: qNope and ctKV int8, kRope and qRope float16/bfloat16")
            _need(cache_mode in (None, MLA_CACHE_KROPE_CTKV), "the int8 cache is a separate (ND) cache")
            for d in (qk_descale, pv_descale):
                _need(d is not None and d.is_cuda and d.dtype == torch.float32 and d.is_contiguous()
                      and d.numel() == q_nope.shape[1], "qk_descale / pv_descale: float32 [headNum] on the device")
        else:
            _need(qk_descale is None and pv_descale is None, "descales go with the int8 cache only")
            _need(dt in _DTYPES and q_nope.dtype == dt and ct_kv.dtype == dt and
                  (k_rope is None or k_rope.dtype == dt), "inputs must share one dtype, float16 or bfloat16")
        _need(q_nope.dim() == 3 and q_nope.shape[2] == 512 and q_rope.shape[:2] == q_nope.shape[:2]
              and q_rope.shape[2] == 64, "qNope [T, H, 512], qRope [T, H, 64]")
        _need(ct_kv.dim() == 4 and ct_kv.shape[2] == 1, "ctKV [numBlocks, blockSize, 1, 512|576]")
        if cache_mode is None:
            cache_mode = MLA_CACHE_KVCACHE if k_rope is None else MLA_CACHE_KROPE_CTKV
        _need(ct_kv.shape[3] == (576 if cache_mode == MLA_CACHE_KVCACHE else 512),
              "ctKV width does not match cacheMode")
        if k_rope is not None:
            _need(k_rope.is_cuda and tuple(k_rope.shape) == (*ct_kv.shape[:3], 64),
                  "kRope [numBlocks, blockSize, 1, 64]")
        _need(all(t is None or t.is_contiguous() for t in (q_nope, q_rope, ct_kv, k_rope, block_tables)),
              "tensors must be contiguous")
        _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2,
              "block_tables must be int32 [batch, maxBlockNum]")
        T, H, _ = q_nope.shape
        self._ctx, p_ctx = _host_i32(context_lens)
        B = len(self._ctx)
        _need(block_tables.shape[0] == B, "block_tables needs one row per sequence")
        if calc_type is None:
            calc_type = MLA_CALC_UNDEFINED if q_seq_len is None else MLA_CALC_SPEC
        if q_seq_len is not None:
            self._ql, p_ql = _host_i32(q_seq_len)
            _need(len(self._ql) == B, "q_seq_len needs one entry per sequence")
            _need(T == int(self._ql.astype(np.int64).sum()), "q_nope has sum(q_seq_len) token rows")
        else:
            self._ql, p_ql = None, ctypes.POINTER(ctypes.c_int32)()
            _need(T == B, "q_nope has one token row per sequence")
        self.out = out if out is not None else torch.empty(q_nope.shape, dtype=dt, device=q_nope.device)
        _need(self.out.shape == q_nope.shape and self.out.dtype == dt and self.out.is_contiguous(),
              "out must be [T, H, 512] of the input dtype")
        if lse is None and return_lse:
            lse = torch.empty((T, H), dtype=torch.float32, device=q_nope.device)
        if lse is not None:
            _need(lse.dtype == torch.float32 and tuple(lse.shape) == (T, H) and lse.is_contiguous(),
                  "lse must be float32 [T, headNum]")
        self.lse = lse
        self._keep = (q_nope, q_rope, ct_kv, k_rope, block_tables, qk_descale, pv_descale)
        self.device = q_nope.device
        ws = ctypes.c_uint64(0)
        op = ctypes.c_void_p(0)
        if quant:
            st = LIB.mpaMLAInt8GetWorkspaceSize(
                _ptr(q_nope), _ptr(q_rope), _ptr(ct_kv), _ptr(k_rope), _ptr(block_tables), p_ctx, p_ql,
                _ptr(qk_descale), _ptr(pv_descale), H, float(qk_scale), 1, int(mask_type), int(calc_type),
                B, ct_kv.shape[0], ct_kv.shape[1], block_tables.shape[1], _DTYPES[dt], T, _ptr(self.out),
                _ptr(lse), ctypes.byref(ws), ctypes.byref(op))
            _check(st, "mpaMLAInt8GetWorkspaceSize")
        else:
            st = LIB.mpaMLAGetWorkspaceSize(
                _ptr(q_nope), _ptr(q_rope), _ptr(ct_kv), _ptr(k_rope), _ptr(block_tables), p_ctx, p_ql,
                H, float(qk_scale), 1, int(mask_type), int(calc_type), int(cache_mode), B,
                ct_kv.shape[0], ct_kv.shape[1], block_tables.shape[1], _DTYPES[dt], T, _ptr(self.out),
                _ptr(lse), ctypes.byref(ws), ctypes.byref(op))
            _check(st, "mpaMLAGetWorkspaceSize")
        self._op = op
        self.workspace = (torch.empty(ws.value, dtype=torch.uint8, device=q_nope.device)
                          if ws.value else None)

    def run(self, stream=None):
        ws = self.workspace
        st = LIB.mpaMLA(_ptr(ws), ws.numel() if ws is not None else 0, self._op,
                        _stream(self.device, stream))
        _check(st, "mpaMLA")
        return (self.out, self.lse) if self.lse is not None else self.out

    def run_static_scratch(self, stream=None):
        """The same launches with the plan and partials in the library's static
        device buffer instead of the workspace (mpaMLAStaticScratch: nothing is
        allocated; executions that overlap on one GPU race)."""
        st = LIB.mpaMLAStaticScratch(self._op, _stream(self.device, stream))
        _check(st, "mpaMLAStaticScratch")
        return (self.out, self.lse) if self.lse is not None else self.out

    def set_launch_events(self, start=None, stop=None):
        """Later runs record ``start`` at the split kernel's start and ``stop`` at the
        end of the call's last kernel (torch.cuda.Event with timing, created, or None)."""
        _set_launch_events(self._op, start, stop)

    def close(self):
        if getattr(self, "_op", None) is not None and self._op.value:
            LIB.mpaDestroyOperation(self._op)
            self._op = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mla(q_nope, q_rope, ct_kv, k_rope, block_tables, context_lens, *, qk_scale, q_seq_len=None,
        mask_type=MLA_MASK_UNDEFINED, calc_type=None, cache_mode=None, out=None, lse=None,
        return_lse=False, stream=None, qk_descale=None, pv_descale=None):
    """One MLA decode call; returns out, or (out, lse) with return_lse."""
    op = MLA(q_nope, q_rope, ct_kv, k_rope, block_tables, context_lens, qk_scale=qk_scale,
             q_seq_len=q_seq_len, mask_type=mask_type, calc_type=calc_type, cache_mode=cache_mode,
             out=out, lse=lse, return_lse=return_lse, qk_descale=qk_descale, pv_descale=pv_descale)
    try:
        return op.run(stream)
    finally:
        torch.cuda.current_stream(q_nope.device).synchronize() if stream is None else stream.synchronize()
        op.close()


def lse_merge(o_parts, lse_parts, *, out=None, lse=None, return_lse=True, stream=None):
    """Merge attention partials over disjoint key ranges by their LSE (mpaLseMerge).

    o_parts [nParts, ..., headDim] float16/bfloat16 and lse_parts [nParts, ...] fp32
    (natural log), e.g. torch.stack of the (out, lse) pairs of several calls over
    disjoint key ranges.  Returns out [..., headDim] (and its LSE with return_lse)."""
    _need(o_parts.dtype in _DTYPES, "o_parts must be float16 or bfloat16")
    _need(lse_parts.dtype == torch.float32, "lse_parts must be float32")
    _need(o_parts.is_cuda and lse_parts.device == o_parts.device, "o_parts and lse_parts on one GPU")
    _need(o_parts.dim() >= 2 and tuple(lse_parts.shape) == tuple(o_parts.shape[:-1]),
          "o_parts [nParts, ..., headDim] and lse_parts [nParts, ...]")
    _need(o_parts.is_contiguous() and lse_parts.is_contiguous(), "parts must be contiguous")
    n_parts, head_dim = o_parts.shape[0], o_parts.shape[-1]
    rows = lse_parts[0].numel() if n_parts else 0
    if out is None:
        out = torch.empty(o_parts.shape[1:], dtype=o_parts.dtype, device=o_parts.device)
    _need(out.dtype == o_parts.dtype and tuple(out.shape) == tuple(o_parts.shape[1:]) and out.is_contiguous(),
          "out must be a contiguous tensor shaped like one part")
    if lse is None and return_lse:
        lse = torch.empty(lse_parts.shape[1:], dtype=torch.float32, device=o_parts.device)
    if lse is not None:
        _need(lse.dtype == torch.float32 and tuple(lse.shape) == tuple(lse_parts.shape[1:]) and lse.is_contiguous(),
              "lse must be a contiguous float32 tensor shaped like one LSE part")
    st = LIB.mpaLseMerge(_ptr(o_parts), _ptr(lse_parts), n_parts, rows, head_dim, _DTYPES[o_parts.dtype],
                         _ptr(out), _ptr(lse), _stream(o_parts.device, stream))
    _check(st, "mpaLseMerge")
    return (out, lse) if lse is not None else out


def plan_prefill(seq_len, kv_seq_len, mask_type, head_num, kv_head_num, head_size=128,
                 with_workspace=False):
    """Host-only view of the prefill launch plan: (items [n, 4] int32 {b, head0, row0,
    n_tiles}, rows_per_item, keys_per_tile, heads_per_item), plus the workspace
    bytes phase 1 returns for it with ``with_workspace``."""
    s, ps = _host_i32(seq_len)
    k, pk = _host_i32(kv_seq_len)
    n = ctypes.c_int64(0)
    rows, keys, heads = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    ws = ctypes.c_uint64(0)
    LIB.mpaPrefixEncoderPlanInspect(ps, pk, len(s), int(mask_type), head_num, kv_head_num, head_size,
                                    ctypes.POINTER(ctypes.c_int32)(), 0, ctypes.byref(n),
                                    ctypes.byref(rows), ctypes.byref(keys), ctypes.byref(heads),
                                    ctypes.byref(ws))
    items = np.zeros((max(1, n.value), 4), dtype=np.int32)
    st = LIB.mpaPrefixEncoderPlanInspect(ps, pk, len(s), int(mask_type), head_num, kv_head_num,
                                         head_size, items.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                         n.value, ctypes.byref(n), ctypes.byref(rows),
                                         ctypes.byref(keys), ctypes.byref(heads), ctypes.byref(ws))
    _check(st, "mpaPrefixEncoderPlanInspect")
    res = (items[:n.value], rows.value, keys.value, heads.value)
    return res + (ws.value,) if with_workspace else res


def plan_mla(context_lens, q_seq_len, head_num, calc_type):
    """Host-only view of the MLA split plan (for 256 compute units): segments
    [n, 5] int32 {b, k0, k1, index among b's segments, piece}, in piece order."""
    c, pc = _host_i32(context_lens)
    if q_seq_len is not None:
        q, pq = _host_i32(q_seq_len)
    else:
        q, pq = None, ctypes.POINTER(ctypes.c_int32)()
    n = ctypes.c_int64(0)
    LIB.mpaMLAPlanInspect(pc, pq, len(c), head_num, int(calc_type), ctypes.POINTER(ctypes.c_int32)(), 0,
                          ctypes.byref(n))
    out = np.zeros((max(1, n.value), 5), dtype=np.int32)
    st = LIB.mpaMLAPlanInspect(pc, pq, len(c), head_num, int(calc_type),
                               out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n.value, ctypes.byref(n))
    _check(st, "mpaMLAPlanInspect")
    return out[:n.value]
