"""Python binding of libtq: an MI355X (gfx950) TurboQuant-style KV codec.

Thin marshalling over the C ABI in include/tq.h: tensors in, tensors out,
launched on torch's current HIP stream.  Every step of encoding, logit
scanning and decoding runs in the library's HIP kernels; PyTorch only
provides device memory and the stream.  There is no CPU fallback: the calls
raise if libtq.so is missing or no GPU is present.

    ck = Codebook(d=128, bits=3, m=64, seed=0)          # keys
    cv = Codebook(d=128, bits=3, m=64, seed=1)          # values

TurboESM-style codebooks (one residual sign per coordinate, a calibrated
mean residual magnitude per KV head, separate key/value tables, values in
their original coordinates):

    lk, mk = calibrate(128, 3, k_sample, seed=0, rope=rope_host)
    lv, mv = calibrate(128, 3, v_sample, rotation="none")
    ck = Codebook(128, 3, 128, seed=0, correction="sign", levels=lk, mu=mk)
    cv = Codebook(128, 3, 128, rotation="none", correction="sign", levels=lv, mu=mv)
    kp, vp = Packed(ck, n), Packed(cv, n)               # n = B * h_kv * L_cap
    encode_kv(ck, cv, k, v, kp, vp, L_cap=L, rope=rope)
    logits = attn_logits(ck, q, kp, h_kv, L, seq_len, rope=rope)
    out = attn_decode(ck, cv, q, kp, vp, h_kv, L, seq_len, rope=rope)
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import _lib
from ._lib import (TQError, TQ_F32, TQ_BF16, TQ_ROT_AUTO, TQ_ROT_HADAMARD, TQ_ROT_DENSE, TQ_ROT_NONE,
                   TQ_CORR_QJL, TQ_CORR_SIGN, TQ_OP_ENCODE, TQ_OP_LOGITS, TQ_OP_DECODE, check, lib, tq_draws,
                   tq_packed, tq_pages, tq_spec)

__all__ = ["Codebook", "Packed", "Pages", "Launch", "encode_kv", "append_kv", "attn_logits", "attn_decode", "attn_decode_noalloc",
           "decode_vectors", "rope_table", "codebook_tables", "plane_words", "workspace_bytes", "calibrate",
           "TQError", "lib"]

_ROT = {"auto": TQ_ROT_AUTO, "hadamard": TQ_ROT_HADAMARD, "dense": TQ_ROT_DENSE, "none": TQ_ROT_NONE}
_CORR = {"qjl": TQ_CORR_QJL, "sign": TQ_CORR_SIGN}


def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _spec(d, bits, m, rotation="auto", seed=0, correction="qjl", block=0):
    return tq_spec(int(d), int(bits), int(m), _ROT[rotation] if isinstance(rotation, str) else int(rotation),
                   int(seed) & 0xFFFFFFFFFFFFFFFF,
                   _CORR[correction] if isinstance(correction, str) else int(correction), int(block))


def _draws(sigma=None, rot_gauss=None, sketch=None):
    keep = []
    dr = tq_draws()
    if sigma is not None:
        a = np.ascontiguousarray(sigma, dtype=np.int8)
        keep.append(a)
        dr.sigma = a.ctypes.data
    if rot_gauss is not None:
        a = np.ascontiguousarray(rot_gauss, dtype=np.float64)
        keep.append(a)
        dr.rot_gauss = a.ctypes.data
    if sketch is not None:
        a = np.ascontiguousarray(sketch, dtype=np.float32)
        keep.append(a)
        dr.sketch = a.ctypes.data
    return dr, keep


def plane_words(d, bits, m, rotation="auto", correction="qjl", block=0):
    """(code words, sign words) per record."""
    sp = _spec(d, bits, m, rotation, 0, correction, block)
    cw = lib().tq_plane_words(C.byref(sp), 0)
    sw = lib().tq_plane_words(C.byref(sp), 1)
    if cw < 0:
        raise TQError(-1, lib().tq_last_error().decode())
    return int(cw), int(sw)


def codebook_tables(d, bits, m, rotation="auto", seed=0, sigma=None, rot_gauss=None, sketch=None,
                    correction="qjl", block=0):
    """Host-only table construction (no GPU): dict of levels (for a vector
    codebook, its codewords [2^bits, block]), thresholds, rotation (sigma as
    +-1 or the dense matrix; zeros for rotation "none") and sketch."""
    sp = _spec(d, bits, m, rotation, seed, correction, block)
    dr, keep = _draws(sigma, rot_gauss, sketch)
    K = 1 << bits
    lv = np.zeros(K * max(1, block), np.float32)
    th = np.zeros(K - 1, np.float32)
    dense = (rotation == "dense") or (rotation == "auto" and (d & (d - 1)) != 0) or rotation == TQ_ROT_DENSE
    rot = np.zeros(d * d if dense else d, np.float32)
    sk = np.zeros(m * d, np.float32)
    check(lib().tq_codebook_tables(C.byref(sp), C.byref(dr), lv.ctypes.data, th.ctypes.data, rot.ctypes.data,
                                   sk.ctypes.data))
    return {"levels": lv.reshape(K, block) if block >= 2 else lv, "thresholds": th,
            "rotation": rot.reshape(d, d) if dense else rot, "sketch": sk.reshape(m, d), "dense": dense}


def calibrate(d, bits, x, rotation="hadamard", seed=0, sigma=None, tok_offset=0, rope=None,
              correction="sign"):
    """Host-only calibration (no GPU) of a table and per-head mean residual
    magnitudes from x [n_tok, h, d] (numpy float32; rope = host (cos, sin)
    tables from rope_table(..., device=None)).  Returns (levels [2^bits],
    mu [h]) as float32 arrays."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n_tok, h, dx = x.shape
    if dx != d:
        raise ValueError("x is [n_tok, h, d]")
    sp = _spec(d, bits, d if correction == "sign" else 0, rotation, seed, correction)
    dr, keep = _draws(sigma, None, None)
    lv = np.zeros(1 << bits, np.float32)
    mu = np.zeros(h, np.float32)
    cs = sn = None
    npos = 0
    if rope is not None:
        cs = np.ascontiguousarray(rope[0], np.float32)
        sn = np.ascontiguousarray(rope[1], np.float32)
        npos = cs.shape[0]
    check(lib().tq_calibrate(C.byref(sp), C.byref(dr), x.ctypes.data, n_tok, h, int(tok_offset),
                             None if cs is None else cs.ctypes.data, None if sn is None else sn.ctypes.data, npos,
                             lv.ctypes.data, mu.ctypes.data))
    return lv, mu


class Codebook:
    """A codebook (Lloyd-Max table, rotation, sketch) resident on the current
    GPU.  Draws default to the library's seeded generator; pass sigma /
    rot_gauss / sketch (host arrays) to supply them.  correction="sign" makes
    a TurboESM-style codebook (m must equal d); levels / mu give a calibrated
    table and per-head mean residual magnitudes (see calibrate).  block=2 or 3
    makes a FibQuant vector codebook of 2^bits codewords per block of that
    many rotated coordinates (m must be 0)."""

    def __init__(self, d, bits, m, rotation="auto", seed=0, sigma=None, rot_gauss=None, sketch=None,
                 correction="qjl", levels=None, mu=None, block=0):
        self.d, self.bits, self.m, self.block = int(d), int(bits), int(m), int(block)
        sp = _spec(d, bits, m, rotation, seed, correction, block)
        dr, keep = _draws(sigma, rot_gauss, sketch)
        lv = None if levels is None else np.ascontiguousarray(levels, np.float32)
        mu_a = None if mu is None else np.ascontiguousarray(np.atleast_1d(mu), np.float32)
        h = C.c_void_p()
        check(lib().tq_codebook_init_calibrated(C.byref(sp), C.byref(dr), None if lv is None else lv.ctypes.data,
                                                None if mu_a is None else mu_a.ctypes.data,
                                                0 if mu_a is None else len(mu_a), _stream(), C.byref(h)))
        self._h = h
        self.correction = correction if isinstance(correction, str) else ("sign" if correction else "qjl")
        self.has_rnorm = self.m > 0 and self.correction == "qjl"
        out = tq_spec()
        check(lib().tq_codebook_get_spec(h, C.byref(out)))
        self.rotation = out.rotation
        self.dense = (out.rotation == TQ_ROT_DENSE) or (out.rotation == TQ_ROT_AUTO and (self.d & (self.d - 1)) != 0)
        self.code_words = int(lib().tq_plane_words(C.byref(sp), 0))
        self.sign_words = self.m // 32

    @property
    def handle(self):
        return self._h

    def mu(self):
        """The mean residual magnitudes (float32 array; empty for the QJL
        sketch)."""
        n = C.c_int32()
        check(lib().tq_codebook_get_mu(self._h, None, C.byref(n)))
        out = np.zeros(n.value, np.float32)
        if n.value:
            check(lib().tq_codebook_get_mu(self._h, out.ctypes.data, C.byref(n)))
        return out

    def export(self):
        K = 1 << self.bits
        lv = np.zeros(K * max(1, self.block), np.float32)
        th = np.zeros(K - 1, np.float32)
        rot = np.zeros(self.d * self.d if self.dense else self.d, np.float32)
        sk = np.zeros(self.m * self.d, np.float32)
        check(lib().tq_codebook_export(self._h, lv.ctypes.data, th.ctypes.data, rot.ctypes.data, sk.ctypes.data))
        return {"levels": lv.reshape(K, self.block) if self.block >= 2 else lv, "thresholds": th,
                "rotation": rot.reshape(self.d, self.d) if self.dense else rot,
                "sketch": sk.reshape(self.m, self.d)}

    def close(self):
        if getattr(self, "_h", None):
            _torch().cuda.synchronize()
            lib().tq_codebook_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            if getattr(self, "_h", None):
                lib().tq_codebook_destroy(self._h)
                self._h = None
        except Exception:
            pass


class Packed:
    """Device planes for n records of one codebook (torch tensors)."""

    def __init__(self, cb: Codebook, n: int, device="cuda"):
        torch = _torch()
        self.n = int(n)
        self.norm = torch.zeros(self.n, dtype=torch.float32, device=device)
        self.rnorm = torch.zeros(self.n if cb.has_rnorm else 0, dtype=torch.float32, device=device)
        self.codes = torch.zeros((self.n, cb.code_words), dtype=torch.int32, device=device)
        self.signs = torch.zeros((self.n, cb.sign_words), dtype=torch.int32, device=device)
        self.m = cb.m
        self.has_rnorm = cb.has_rnorm

    @classmethod
    def from_arrays(cls, cb, norm, rnorm, codes, signs, device="cuda"):
        torch = _torch()
        p = cls.__new__(cls)
        p.n = int(len(norm))
        p.m = cb.m
        p.has_rnorm = cb.has_rnorm
        p.norm = torch.as_tensor(np.asarray(norm, np.float32), device=device)
        p.rnorm = torch.as_tensor(np.asarray(rnorm if cb.has_rnorm else np.zeros(0), np.float32), device=device)
        p.codes = torch.as_tensor(np.asarray(codes, np.uint32).view(np.int32), device=device)
        p.signs = torch.as_tensor(np.asarray(signs if cb.m else np.zeros((p.n, 0)), np.uint32).view(np.int32),
                                  device=device)
        return p

    def struct(self):
        return tq_packed(self.norm.data_ptr(), self.rnorm.data_ptr() if self.has_rnorm else None, self.codes.data_ptr(),
                         self.signs.data_ptr() if self.m else None, self.n)

    def numpy(self):
        """(norm, rnorm, codes uint32, signs uint32) on the host."""
        return (self.norm.cpu().numpy(), self.rnorm.cpu().numpy(),
                self.codes.cpu().numpy().view(np.uint32), self.signs.cpu().numpy().view(np.uint32))


class Pages:
    """A page table for paged records: table int32 [B, max_pages] on the GPU
    (physical page of each sequence's logical page), pages of page_size
    slots (a multiple of 64), n_pages physical pages in the pool.  Record
    planes for it hold records(h_kv) records."""

    def __init__(self, table, page_size, n_pages):
        torch = _torch()
        if table.dtype != torch.int32 or table.dim() != 2 or not table.is_contiguous():
            raise ValueError("the page table is a contiguous int32 [B, max_pages] tensor")
        self.table = table
        self.page_size = int(page_size)
        self.n_pages = int(n_pages)
        self.max_pages = int(table.shape[1])

    @property
    def capacity(self):
        """Logical slots per sequence."""
        return self.max_pages * self.page_size

    def records(self, h_kv):
        return self.n_pages * int(h_kv) * self.page_size

    def struct(self):
        return tq_pages(self.table.data_ptr(), self.page_size, self.max_pages, self.n_pages)


class Launch:
    """One library call with its arguments marshalled once: calling it
    enqueues the same work again (same buffers, sizes and stream).  Loops that
    repeat a call (a layer's encode, a decode step) pay the Python-side
    argument handling once instead of per launch."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep  # host objects the pointers in args refer to

    def __call__(self):
        code = self._fn(*self._args)
        if code != 0:
            raise TQError(code, lib().tq_last_error().decode())


def _run(fn, args, keep, prepare):
    if prepare:
        return Launch(fn, tuple(args), keep)
    check(fn(*args))
    return None


def decode_vectors(cb, packed, first=0, count=None, out=None):
    """The vector codebook's decoder: records [first, first + count) rebuilt
    as float32 [count, d] (nu Pi^T of the looked-up codewords)."""
    torch = _torch()
    count = packed.n - first if count is None else int(count)
    if out is None:
        out = torch.empty((count, cb.d), dtype=torch.float32, device="cuda")
    pst = packed.struct()
    check(lib().tq_decode_vectors(cb.handle, C.byref(pst), int(first), count, _ptr(out), _stream()))
    return out


def workspace_bytes(ck, cv, op, B, Hq=0, h_kv=1, L_cap=0, top_k=0):
    return int(lib().tq_workspace_bytes(ck.handle, cv.handle if cv else None, op, int(B), int(Hq), int(h_kv),
                                        int(L_cap), int(top_k)))


def _workspace(nbytes):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device="cuda"), nbytes


def rope_table(base, d, n_pos, device="cuda"):
    """(cos, sin) float32 [n_pos, d/2] from the library's host builder, on
    ``device`` (or numpy arrays if device is None)."""
    cs = np.zeros((n_pos, d // 2), np.float32)
    sn = np.zeros((n_pos, d // 2), np.float32)
    check(lib().tq_rope_table(float(base), int(d), int(n_pos), cs.ctypes.data, sn.ctypes.data))
    if device is None:
        return cs, sn
    torch = _torch()
    return torch.as_tensor(cs, device=device), torch.as_tensor(sn, device=device)


def _strides(t):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("inputs are [n_seq, n_tok, h_kv, d] with d contiguous")
    return (C.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def encode_kv(ck, cv, k, v, kout=None, vout=None, tok_offset=0, L_cap=None, rope=None, workspace=None,
              prepare=False, pages=None):
    """Encode k and/or v ([n_seq, n_tok, h_kv, d], float32 or bfloat16) into
    Packed planes at cache slots tok_offset.. of each (seq, head) (through
    the page table when pages is a Pages).  With prepare=True nothing runs:
    a Launch that enqueues this call is returned (the tensors must stay alive
    and in place)."""
    x = k if k is not None else v
    n_seq, n_tok, h_kv, _ = x.shape
    if pages is not None:
        ks = _strides(k) if k is not None else None
        vs = _strides(v) if v is not None else None
        cos, sin = (None, None) if rope is None else rope
        npos = 0 if rope is None else int(cos.shape[0])
        pst = pages.struct()
        kst = kout.struct() if kout is not None else None
        vst = vout.struct() if vout is not None else None
        args = [ck.handle if ck else None, cv.handle if cv else None, _ptr(k), _ptr(v), _dtype_code(x), n_seq, n_tok,
                h_kv, ks, vs, int(tok_offset), C.byref(pst), _ptr(cos), _ptr(sin), npos,
                C.byref(kst) if kst is not None else None, C.byref(vst) if vst is not None else None, _stream()]
        launch = _run(lib().tq_encode_kv_paged, args, (kst, vst, ks, vs, pst), prepare)
        return launch if prepare else (kout, vout)
    L_cap = n_tok + tok_offset if L_cap is None else int(L_cap)
    dt = _dtype_code(x)
    ks = _strides(k) if k is not None else None
    vs = _strides(v) if v is not None else None
    need = workspace_bytes(ck if k is not None else cv, cv if (k is not None and v is not None) else None,
                           TQ_OP_ENCODE, n_seq * n_tok * h_kv)
    ws, wsb = (workspace, workspace.numel()) if workspace is not None else _workspace(need)
    cos, sin = (None, None) if rope is None else rope
    npos = 0 if rope is None else int(cos.shape[0])
    kst = kout.struct() if kout is not None else None
    vst = vout.struct() if vout is not None else None
    args = [ck.handle if ck else None, cv.handle if cv else None, _ptr(k), _ptr(v), dt, n_seq, n_tok, h_kv, ks, vs,
            int(tok_offset), L_cap, _ptr(cos), _ptr(sin), npos, C.byref(kst) if kst is not None else None,
            C.byref(vst) if vst is not None else None, _ptr(ws), wsb, _stream()]
    launch = _run(lib().tq_encode_kv, args, (kst, vst, ks, vs, ws), prepare)
    return launch if prepare else (kout, vout)


def append_kv(ck, cv, k, v, kout, vout, pos, pages=None, L_cap=None, rope=None, prepare=False):
    """One autoregressive step: k and/or v [B, h_kv, d] (float32 or bfloat16),
    the token of sequence b written at slot pos[b] (int32 [B] on the GPU),
    through the page table when pages is given, else into contiguous records
    of L_cap slots."""
    x = k if k is not None else v
    B, h_kv, _ = x.shape

    def strides(t):
        if t is None:
            return None
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError("append inputs are [B, h_kv, d] with d contiguous")
        return (C.c_int64 * 2)(t.stride(0), t.stride(1))
    ks, vs = strides(k), strides(v)
    cos, sin = (None, None) if rope is None else rope
    npos = 0 if rope is None else int(cos.shape[0])
    pst = pages.struct() if pages is not None else None
    kst = kout.struct() if kout is not None else None
    vst = vout.struct() if vout is not None else None
    args = [ck.handle if ck else None, cv.handle if cv else None, _ptr(k), _ptr(v), _dtype_code(x), B, h_kv, ks, vs,
            _ptr(pos), C.byref(pst) if pst is not None else None, 0 if L_cap is None else int(L_cap), _ptr(cos),
            _ptr(sin), npos, C.byref(kst) if kst is not None else None, C.byref(vst) if vst is not None else None,
            _stream()]
    return _run(lib().tq_append_kv, args, (kst, vst, ks, vs, pst), prepare)


def attn_logits(ck, q, kp, h_kv, L_cap, seq_len, rope=None, top_k=0, out=None, workspace=None, prepare=False,
                pages=None, q_pos=None):
    """Logits [B, Hq, L_cap] (top_k = 0) or (values, indices) [B, Hq, top_k]
    for queries q [B, Hq, d] against packed keys.  seq_len: int32 [B] on the
    GPU; q_pos: int32 [B] on the GPU, the queries' RoPE positions (None:
    seq_len).  With pages (a Pages), keys are read through the page table and
    L_cap is its capacity.  prepare=True returns (Launch, outputs) without
    running."""
    torch = _torch()
    B, Hq, d = q.shape
    if pages is not None:
        L_cap = pages.capacity
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    cos, sin = (None, None) if rope is None else rope
    npos = 0 if rope is None else int(cos.shape[0])
    need = workspace_bytes(ck, None, TQ_OP_LOGITS, B, Hq, h_kv, L_cap, top_k)
    ws, wsb = (workspace, workspace.numel()) if workspace is not None else _workspace(need)
    idx = None
    if top_k:
        out = torch.empty((B, Hq, top_k), dtype=torch.float32, device=q.device) if out is None else out
        idx = torch.empty((B, Hq, top_k), dtype=torch.int32, device=q.device)
    elif out is None:
        out = torch.zeros((B, Hq, L_cap), dtype=torch.float32, device=q.device)
    kst = kp.struct()
    if pages is not None:
        pst = pages.struct()
        args = [ck.handle, _ptr(q), _dtype_code(q), C.byref(kst), B, Hq, int(h_kv), _ptr(seq_len), _ptr(q_pos),
                C.byref(pst), _ptr(cos), _ptr(sin), npos, int(top_k), _ptr(out), _ptr(idx), _ptr(ws), wsb, _stream()]
        launch = _run(lib().tq_attn_logits_paged, args, (kst, pst, ws, out, idx), prepare)
    else:
        args = [ck.handle, _ptr(q), _dtype_code(q), C.byref(kst), B, Hq, int(h_kv), int(L_cap), _ptr(seq_len),
                _ptr(q_pos), _ptr(cos), _ptr(sin), npos, int(top_k), _ptr(out), _ptr(idx), _ptr(ws), wsb, _stream()]
        launch = _run(lib().tq_attn_logits, args, (kst, ws, out, idx), prepare)
    res = (out, idx) if top_k else out
    return (launch, res) if prepare else res


def attn_decode(ck, cv, q, kp, vp, h_kv, L_cap, seq_len, rope=None, scale=0.0, out=None, workspace=None,
                prepare=False, pages=None, q_pos=None):
    """Decode attention output [B, Hq, d] float32 over packed K and V (read
    through the page table when pages is given; L_cap is then its capacity).
    q_pos: the queries' RoPE positions (int32 [B] on the GPU; None: seq_len).
    prepare=True returns (Launch, out) without running."""
    torch = _torch()
    B, Hq, d = q.shape
    if pages is not None:
        L_cap = pages.capacity
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    cos, sin = (None, None) if rope is None else rope
    npos = 0 if rope is None else int(cos.shape[0])
    need = workspace_bytes(ck, cv, TQ_OP_DECODE, B, Hq, h_kv, L_cap, 0)
    ws, wsb = (workspace, workspace.numel()) if workspace is not None else _workspace(need)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    kst, vst = kp.struct(), vp.struct()
    if pages is not None:
        pst = pages.struct()
        args = [ck.handle, cv.handle, _ptr(q), _dtype_code(q), C.byref(kst), C.byref(vst), B, Hq, int(h_kv),
                _ptr(seq_len), _ptr(q_pos), C.byref(pst), _ptr(cos), _ptr(sin), npos, float(scale), _ptr(out),
                _ptr(ws), wsb, _stream()]
        launch = _run(lib().tq_attn_decode_paged, args, (kst, vst, pst, ws, out), prepare)
    else:
        args = [ck.handle, cv.handle, _ptr(q), _dtype_code(q), C.byref(kst), C.byref(vst), B, Hq, int(h_kv),
                int(L_cap), _ptr(seq_len), _ptr(q_pos), _ptr(cos), _ptr(sin), npos, float(scale), _ptr(out),
                _ptr(ws), wsb, _stream()]
        launch = _run(lib().tq_attn_decode, args, (kst, vst, ws, out), prepare)
    return (launch, out) if prepare else out


def attn_decode_noalloc(ck, cv, q, kp, vp, h_kv, L_cap, seq_len, rope=None, scale=0.0, out=None, prepare=False,
                        q_pos=None):
    """attn_decode with the library's static device scratch as its workspace
    (the library allocates nothing; out is allocated here when not given).
    Calls that overlap on one GPU race on that scratch."""
    torch = _torch()
    B, Hq, d = q.shape
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    cos, sin = (None, None) if rope is None else rope
    npos = 0 if rope is None else int(cos.shape[0])
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    kst, vst = kp.struct(), vp.struct()
    args = [ck.handle, cv.handle, _ptr(q), _dtype_code(q), C.byref(kst), C.byref(vst), B, Hq, int(h_kv),
            int(L_cap), _ptr(seq_len), _ptr(q_pos), _ptr(cos), _ptr(sin), npos, float(scale), _ptr(out), _stream()]
    launch = _run(lib().tq_attn_decode_noalloc, args, (kst, vst, out), prepare)
    return (launch, out) if prepare else out
