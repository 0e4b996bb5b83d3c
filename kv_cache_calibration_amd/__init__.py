"""NSNQuant KV-cache quantization for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libnsn.so`` (include/nsn.h): every
function here only marshals torch device tensors into pointers, sizes and
strides and calls the function of the same name; all computation runs in the
library's HIP kernels on the caller's current HIP stream.

Tensor conventions (dim 0 is always the flattened sequence axis; inner dims
must be contiguous):
    x       (n_seq, n_tok, 128)            fp16 or fp32
    codes   (n_seq, cap, 128 // m)         uint8
    meta    (n_seq, cap, 2)                fp16   (s1, s2')
    shift   (n_seq, cap // G, 128)         fp16   rotated group mean
    table   (nsn_table_size,)              uint8  prepared codebook
With double quantization (``Params(dq=True)``, NSN_DQ, G = 128):
    meta    (n_seq, cap)                   fp16   s2'
    shift   (n_seq, cap // 128, 136)       uint8  group records
            (any 2-byte-aligned dtype works; strides are passed in bytes / 2)
"""

import ctypes

from . import _lib
from ._lib import NSN_DQ, NSN_RHT, NSN_SCALE_ADJUST, NsnError  # noqa: F401

__all__ = [
    "Params",
    "NsnError",
    "nsn_table_size",
    "nsn_build_codebook",
    "nsn_tune_codebook",
    "nsn_tune_codebook_workspace_size",
    "nsn_prepare_codebook",
    "nsn_nearest_codeword",
    "nsn_quantize",
    "nsn_dequantize",
    "nsn_residual_append",
    "nsn_decode_attention",
    "nsn_decode_attention_rope",
    "nsn_decode_attention_noalloc",
    "nsn_decode_attention_workspace_size",
    "PreparedDecodeAttention",
    "PreparedResidualAppend",
    "lib_path",
    "cache_layout",
]


def lib_path():
    return _lib.LIB_PATH


class Params:
    """Python view of ``nsn_params``.

    ``rht_signs``: None for the plain Hadamard rotation, or head_dim values
    of +1 / -1 (channel c negated before the transform where it is -1),
    packed into the NSN_RHT bit mask."""

    def __init__(self, sub_dim=4, group_size=128, scale_adjust=True, head_dim=128, n_codes=256,
                 dq=False, rht_signs=None):
        flags = (NSN_SCALE_ADJUST if scale_adjust else 0) | (NSN_DQ if dq else 0)
        words = [0, 0, 0, 0]
        if rht_signs is not None:
            signs = [float(v) for v in rht_signs]
            if len(signs) != 128 or any(v not in (1.0, -1.0) for v in signs):
                raise ValueError("rht_signs must be 128 values of +1 or -1")
            for c, v in enumerate(signs):
                if v < 0:
                    words[c // 32] |= 1 << (c % 32)
            flags |= NSN_RHT
        self.c = _lib.nsn_params(head_dim, sub_dim, n_codes, group_size, flags,
                                 (ctypes.c_uint32 * 4)(*words))

    @property
    def sub_dim(self):
        return self.c.sub_dim

    @property
    def group_size(self):
        return self.c.group_size

    @property
    def dq(self):
        return bool(self.c.flags & NSN_DQ)

    @property
    def rht(self):
        return bool(self.c.flags & NSN_RHT)


def _stride16(t):
    """dim-0 stride in 2-byte units (meta and shift strides of the C ABI)."""
    b = t.stride(0) * t.element_size()
    if b % 2:
        raise ValueError("meta and shift sequence strides must be a whole number of 2-byte units")
    return b // 2


def _check_meta_layout(params, meta, shift):
    """Inner shapes of meta and shift for the plain and the double-quantized
    layouts (see the module doc)."""
    import torch
    if meta.dtype != torch.float16:
        raise ValueError("meta must be fp16")
    if params.dq:
        if meta.dim() != 2 or meta.element_size() != 2:
            raise ValueError("with dq, meta is (n_seq, cap) of a 2-byte dtype (fp16 s2')")
        if shift.dim() != 3 or shift.shape[2] * shift.element_size() != 136:
            raise ValueError("with dq, shift is (n_seq, cap // 128, 136 bytes) of group records")
    else:
        if meta.dim() != 3 or meta.shape[2] != 2 or meta.element_size() != 2:
            raise ValueError("meta is (n_seq, cap, 2) fp16")
        if shift.dim() != 3 or shift.shape[2] != 128 or shift.dtype != torch.float16:
            raise ValueError("shift is (n_seq, cap // G, 128) fp16")


def _check_extents(params, n_seq, n_tok, codes, meta, shift):
    """Every output/input array holds n_seq sequences of n_tok tokens
    (n_tok / G group slots for shift): the C ABI trusts these extents."""
    for name, t in (("codes", codes), ("meta", meta), ("shift", shift)):
        if t.shape[0] < n_seq:
            raise ValueError(f"{name} has {t.shape[0]} sequences, fewer than {n_seq}")
    if codes.shape[1] < n_tok or meta.shape[1] < n_tok:
        raise ValueError("n_tok exceeds the tensors' token dimension")
    if shift.shape[1] < n_tok // params.group_size:
        raise ValueError(f"shift holds {shift.shape[1]} group slots, fewer than "
                         f"n_tok // group_size = {n_tok // params.group_size}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


_raw_stream = None


def _stream(stream):
    """HIP stream handle of the call: the given torch stream, else torch's
    current stream on the current device.  The latter is read through
    torch's raw getter when it exists (building a Stream object costs more
    than the kernel launch of a small call)."""
    global _raw_stream
    import torch
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if _raw_stream is None:
        getter = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if getter is not None:
            _raw_stream = lambda: getter(torch.cuda.current_device())  # noqa: E731
        else:
            _raw_stream = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731
    return ctypes.c_void_p(_raw_stream())


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be HIP device tensors")


def _inner_contig(t, inner):
    """dims >= 1 contiguous with the given inner sizes."""
    if inner is not None and tuple(t.shape[1:]) != tuple(inner):
        raise ValueError(f"expected inner shape {inner}, got {tuple(t.shape[1:])}")
    st = 1
    for d in range(t.dim() - 1, 0, -1):
        if t.shape[d] > 1 and t.stride(d) != st:
            raise ValueError("inner dimensions must be contiguous")
        st *= t.shape[d]


def cache_layout(params, n_seq, cap):
    """Shapes and torch dtypes of (codes, meta, shift) for n_seq sequences of
    cap token slots in the layout ``params`` selects (plain or double
    quantized); cap is a multiple of the group size."""
    import torch
    G, m = params.group_size, params.sub_dim
    if cap % G:
        raise ValueError("cap must be a multiple of group_size")
    codes = ((n_seq, cap, 128 // m), torch.uint8)
    if params.dq:
        return codes, ((n_seq, cap), torch.float16), ((n_seq, cap // G, 136), torch.uint8)
    return codes, ((n_seq, cap, 2), torch.float16), ((n_seq, cap // G, 128), torch.float16)


def nsn_table_size(params):
    return int(_lib.load().nsn_table_size(ctypes.byref(params.c)))


def nsn_build_codebook(samples, codebook, workspace, iters=20, n_codes=256, stream=None):
    """samples float64 (n, m) device; codebook float32 (n_codes, m) device (written)."""
    import torch
    _dev(samples, codebook, workspace)
    if samples.dtype != torch.float64 or codebook.dtype != torch.float32:
        raise ValueError("samples must be float64 and codebook float32")
    if not samples.is_contiguous() or not codebook.is_contiguous():
        raise ValueError("samples and codebook must be contiguous")
    lib = _lib.load()
    _lib.check(lib.nsn_build_codebook(samples.shape[1], n_codes, samples.shape[0], iters,
                                      _ptr(samples), _ptr(codebook), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream)))


def nsn_tune_codebook(vectors, codebook, workspace, iters, lr=1e-3, n_codes=256, stream=None):
    """vectors float64 (n_vec, 128) device; codebook float32 (n_codes, m) device,
    the start on entry and the tuned, fp16-rounded codebook on return."""
    import torch
    _dev(vectors, codebook, workspace)
    if vectors.dtype != torch.float64 or codebook.dtype != torch.float32:
        raise ValueError("vectors must be float64 and codebook float32")
    if not vectors.is_contiguous() or not codebook.is_contiguous() or vectors.shape[1] != 128:
        raise ValueError("vectors (n, 128) and codebook must be contiguous")
    lib = _lib.load()
    _lib.check(lib.nsn_tune_codebook(codebook.shape[1], n_codes, vectors.shape[0], iters, lr,
                                     _ptr(vectors), _ptr(codebook), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))


def nsn_tune_codebook_workspace_size(sub_dim, n_vec, n_codes=256):
    return int(_lib.load().nsn_tune_codebook_workspace_size(sub_dim, n_codes, n_vec))


def nsn_build_codebook_workspace_size(sub_dim, n_samples, n_codes=256):
    return int(_lib.load().nsn_build_codebook_workspace_size(sub_dim, n_codes, n_samples))


def nsn_prepare_codebook(params, codebook, table, stream=None):
    """Prepare `table` from `codebook` for `params`.  The tensor remembers the
    sub-vector size and metadata layout it was prepared for (its contents
    depend on both), and every call of this module that takes the table
    refuses params that differ."""
    _dev(codebook, table)
    _lib.check(_lib.load().nsn_prepare_codebook(ctypes.byref(params.c), _ptr(codebook),
                                                _ptr(table), table.numel() * table.element_size(),
                                                _stream(stream)))
    table._nsn_prepared_for = _table_key(params)


def nsn_nearest_codeword(params, table, v, out, stream=None):
    """Nearest codeword index of every row of v (float32 (n, sub_dim)) -> out uint8 (n,)."""
    import torch
    _dev(table, v, out)
    if v.dtype != torch.float32 or out.dtype != torch.uint8:
        raise ValueError("v must be float32 and out uint8")
    if not v.is_contiguous() or not out.is_contiguous() or v.shape[-1] != params.sub_dim:
        raise ValueError("v must be contiguous (n, sub_dim) and out contiguous (n,)")
    n = v.numel() // params.sub_dim
    if out.numel() < n:
        raise ValueError("out too small")
    _check_table(params, table)
    _lib.check(_lib.load().nsn_nearest_codeword(ctypes.byref(params.c), _ptr(table), _ptr(v), n,
                                                _ptr(out), _stream(stream)))


def _table_key(params):
    return (params.sub_dim, params.dq)


def _check_table(params, table):
    if table.numel() * table.element_size() < nsn_table_size(params):
        raise ValueError("table is smaller than nsn_table_size(params)")
    made_for = getattr(table, "_nsn_prepared_for", None)
    if made_for is not None and made_for != _table_key(params):
        raise ValueError(f"table was prepared for (sub_dim, dq) = {made_for}, "
                         f"used with {_table_key(params)}")


def _check_codes(params, codes):
    import torch
    if codes.dtype != torch.uint8 or codes.shape[-1] != 128 // params.sub_dim:
        raise ValueError(f"codes must be uint8 with {128 // params.sub_dim} bytes per token")


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return _lib.NSN_F16
    if t.dtype == torch.float32:
        return _lib.NSN_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def nsn_quantize(params, x, table, codes, meta, shift, n_tok=None, stream=None):
    """Quantize x (n_seq, n_tok, 128) into codes/meta/shift (see module doc).

    The output tensors may be views into a larger cache (e.g. advanced to a
    group offset); their dim-0 strides are passed through."""
    _dev(x, table, codes, meta, shift)
    n_tok = x.shape[1] if n_tok is None else n_tok
    _inner_contig(x, (x.shape[1], 128))
    _inner_contig(codes, None)
    _inner_contig(meta, None)
    _inner_contig(shift, None)
    _check_meta_layout(params, meta, shift)
    _check_codes(params, codes)
    _check_table(params, table)
    if x.shape[1] < n_tok:
        raise ValueError("n_tok exceeds the input's token dimension")
    _check_extents(params, x.shape[0], n_tok, codes, meta, shift)
    lib = _lib.load()
    _lib.check(lib.nsn_quantize(ctypes.byref(params.c), _dtype_code(x), _ptr(x), x.shape[0], n_tok,
                                x.stride(0), _ptr(table), _ptr(codes), codes.stride(0), _ptr(meta),
                                _stride16(meta), _ptr(shift), _stride16(shift), _stream(stream)))


def nsn_dequantize(params, codes, meta, shift, table, out, n_tok=None, stream=None):
    _dev(codes, meta, shift, table, out)
    n_tok = out.shape[1] if n_tok is None else n_tok
    _inner_contig(out, (out.shape[1], 128))
    _inner_contig(codes, None)
    _inner_contig(meta, None)
    _inner_contig(shift, None)
    _check_meta_layout(params, meta, shift)
    _check_codes(params, codes)
    _check_table(params, table)
    if out.shape[1] < n_tok:
        raise ValueError("n_tok exceeds the output's token dimension")
    _check_extents(params, out.shape[0], n_tok, codes, meta, shift)
    lib = _lib.load()
    _lib.check(lib.nsn_dequantize(ctypes.byref(params.c), _ptr(codes), codes.stride(0), _ptr(meta),
                                  _stride16(meta), _ptr(shift), _stride16(shift), _ptr(table),
                                  out.shape[0], n_tok, _dtype_code(out), _ptr(out), out.stride(0),
                                  _stream(stream)))


def _check_append(tok, resid):
    _dev(tok, resid)
    import torch
    if not tok.is_contiguous():
        raise ValueError("tok must be contiguous")
    if tok.dtype != torch.float16 or resid.dtype != torch.float16 or tuple(tok.shape) != (resid.shape[0], 128):
        raise ValueError("tok must be fp16 (n_seq, 128) and resid fp16 (n_seq, cap, 128)")
    _inner_contig(resid, (resid.shape[1], 128))


def nsn_residual_append(tok, resid, pos, stream=None):
    """tok fp16 (n_seq, 128); resid fp16 (n_seq, cap, 128)."""
    _check_append(tok, resid)
    lib = _lib.load()
    _lib.check(lib.nsn_residual_append(_ptr(tok), tok.shape[0], _ptr(resid), resid.stride(0),
                                       resid.shape[1], pos, _stream(stream)))


class PreparedResidualAppend:
    """nsn_residual_append with its tensors checked and marshalled once, for a
    decode loop that writes each step's token into the same buffer `tok`.
    Calling the object with the step's residual slot makes the library call
    (which still validates every argument); the object holds references to
    the tensors, which must keep their shapes.  Results equal those of the
    per-call function."""

    def __init__(self, tok, resid):
        _check_append(tok, resid)
        self._keep = (tok, resid)
        self._fn = _lib.load().nsn_residual_append
        self._head = (_ptr(tok), tok.shape[0], _ptr(resid), resid.stride(0), resid.shape[1])

    def __call__(self, pos, stream=None):
        status = self._fn(*self._head, pos, _stream(stream))
        if status != _lib.NSN_OK:
            _lib.check(status)


def _shape(batch, n_q_heads, n_kv_heads, n_quant_tok, n_resid_tok, cache_capacity,
           resid_capacity, softmax_scale):
    return _lib.nsn_attn_shape(batch, n_q_heads, n_kv_heads, n_quant_tok, n_resid_tok,
                               cache_capacity, resid_capacity, softmax_scale)


def nsn_decode_attention_workspace_size(params, batch, n_q_heads, n_kv_heads, n_quant_tok,
                                        n_resid_tok, cache_capacity, resid_capacity,
                                        softmax_scale):
    s = _shape(batch, n_q_heads, n_kv_heads, n_quant_tok, n_resid_tok, cache_capacity,
               resid_capacity, softmax_scale)
    return int(_lib.load().nsn_decode_attention_workspace_size(ctypes.byref(params.c),
                                                               ctypes.byref(s)))


def nsn_decode_attention_rope(params, q, k_cache, v_cache, k_resid, v_resid, table, workspace,
                              out, n_quant_tok, n_resid_tok, softmax_scale, q_pos, rope_base,
                              stream=None):
    """nsn_decode_attention for keys stored before rotary embedding: the query
    (at q_pos) and every key (quantized key t at position t, residual key r at
    n_quant_tok + r) are turned by the rotate-half rotary embedding with the
    given base.  Same tensors as nsn_decode_attention."""
    _decode_attention(params, q, k_cache, v_cache, k_resid, v_resid, table, workspace, out,
                      n_quant_tok, n_resid_tok, softmax_scale, stream,
                      _lib.nsn_rope(int(q_pos), float(rope_base)))


def nsn_decode_attention(params, q, k_cache, v_cache, k_resid, v_resid, table, workspace, out,
                         n_quant_tok, n_resid_tok, softmax_scale, stream=None):
    """q fp16 (B, Hq, 128); k_cache/v_cache = (codes (B, Hkv, cap, 128/m) uint8,
    meta (B, Hkv, cap, 2) fp16, shift (B, Hkv, cap/G, 128) fp16), all contiguous;
    k_resid/v_resid fp16 (B, Hkv, Rcap, 128) contiguous; out fp32 (B, Hq, 128)."""
    _decode_attention(params, q, k_cache, v_cache, k_resid, v_resid, table, workspace, out,
                      n_quant_tok, n_resid_tok, softmax_scale, stream, None)


def nsn_decode_attention_noalloc(params, q, k_cache, v_cache, k_resid, v_resid, table, out,
                                 n_quant_tok, n_resid_tok, softmax_scale, stream=None):
    """nsn_decode_attention without a workspace: the library's static device
    scratch holds the split partials (calls on one GPU must not overlap)."""
    _decode_attention(params, q, k_cache, v_cache, k_resid, v_resid, table, None, out,
                      n_quant_tok, n_resid_tok, softmax_scale, stream, None, noalloc=True)


def _check_attention_shapes(params, q, k_cache, v_cache, k_resid, v_resid, out):
    """The sizes the C ABI derives from the shape struct must match the
    tensors: q and out (B, Hq, 128), codes (B, Hkv, cap, 128 // m), meta
    and shift per layout, residuals (B, Hkv, Rcap, 128)."""
    B, Hq = q.shape[0], q.shape[1]
    kc = k_cache[0]
    Hkv, cap = kc.shape[1], kc.shape[2]
    G = params.group_size
    import torch
    if tuple(q.shape) != (B, Hq, 128) or tuple(out.shape) != (B, Hq, 128):
        raise ValueError("q and out must be (B, Hq, 128)")
    if q.dtype != torch.float16 or out.dtype != torch.float32:
        raise ValueError("q must be fp16 and out fp32")
    if k_resid.dtype != torch.float16 or v_resid.dtype != torch.float16:
        raise ValueError("residuals must be fp16")
    for c, mt, sh in (k_cache, v_cache):
        if tuple(c.shape) != (B, Hkv, cap, 128 // params.sub_dim) or c.dtype != torch.uint8:
            raise ValueError("codes must be (B, Hkv, cap, 128 // m), alike for K and V")
        if params.dq:
            ok = (tuple(mt.shape) == (B, Hkv, cap) and mt.element_size() == 2 and
                  tuple(sh.shape[:3]) == (B, Hkv, cap // G) and sh.dim() == 4 and
                  sh.shape[3] * sh.element_size() == 136)
        else:
            ok = (tuple(mt.shape) == (B, Hkv, cap, 2) and mt.element_size() == 2 and
                  tuple(sh.shape) == (B, Hkv, cap // G, 128) and sh.element_size() == 2)
        if not ok:
            raise ValueError("meta / shift shapes do not match the cache layout")
    for r in (k_resid, v_resid):
        if r.dim() != 4 or tuple(r.shape[:2]) != (B, Hkv) or r.shape[3] != 128 or r.shape != k_resid.shape:
            raise ValueError("residuals must be (B, Hkv, Rcap, 128), alike for K and V")


def _check_attention_call(params, q, k_cache, v_cache, k_resid, v_resid, table, workspace, out):
    kc, km, ks = k_cache
    vc, vm, vs = v_cache
    _dev(q, kc, km, ks, vc, vm, vs, k_resid, v_resid, table, workspace, out)
    for t in (q, kc, km, ks, vc, vm, vs, k_resid, v_resid, out):
        if not t.is_contiguous():
            raise ValueError("attention tensors must be contiguous")
    _check_attention_shapes(params, q, k_cache, v_cache, k_resid, v_resid, out)
    _check_table(params, table)


def _decode_attention(params, q, k_cache, v_cache, k_resid, v_resid, table, workspace, out,
                      n_quant_tok, n_resid_tok, softmax_scale, stream, rope, noalloc=False):
    kc, km, ks = k_cache
    vc, vm, vs = v_cache
    _check_attention_call(params, q, k_cache, v_cache, k_resid, v_resid, table, workspace, out)
    B, Hq, _ = q.shape
    Hkv, cap = kc.shape[1], kc.shape[2]
    s = _shape(B, Hq, Hkv, n_quant_tok, n_resid_tok, cap, k_resid.shape[2], softmax_scale)
    lib = _lib.load()
    if noalloc:
        _lib.check(lib.nsn_decode_attention_noalloc(
            ctypes.byref(params.c), ctypes.byref(s), _ptr(q), _ptr(kc), _ptr(km), _ptr(ks), _ptr(vc),
            _ptr(vm), _ptr(vs), _ptr(k_resid), _ptr(v_resid), _ptr(table), _ptr(out), _stream(stream)))
        return
    bufs = (_ptr(q), _ptr(kc), _ptr(km), _ptr(ks), _ptr(vc), _ptr(vm), _ptr(vs), _ptr(k_resid),
            _ptr(v_resid), _ptr(table), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream))
    if rope is None:
        _lib.check(lib.nsn_decode_attention(ctypes.byref(params.c), ctypes.byref(s), *bufs))
    else:
        _lib.check(lib.nsn_decode_attention_rope(ctypes.byref(params.c), ctypes.byref(s),
                                                 ctypes.byref(rope), *bufs))


class PreparedDecodeAttention:
    """nsn_decode_attention -- or nsn_decode_attention_rope when ``rope_base``
    is given -- with its tensors checked and marshalled once, for a decode
    loop that passes the same buffers every step.

    Calling the object with the step's token counts (and the query position
    for rotary keys) sets them in the shape struct and makes the library
    call, which still validates every argument; the tensors' devices,
    dtypes, shapes and contiguity are checked here once, so they must keep
    their shapes afterwards (the object holds references to them, so they
    stay allocated).  Results equal those of the per-call function."""

    def __init__(self, params, q, k_cache, v_cache, k_resid, v_resid, table, workspace, out,
                 softmax_scale, rope_base=None):
        _check_attention_call(params, q, k_cache, v_cache, k_resid, v_resid, table, workspace, out)
        kc, km, ks = k_cache
        vc, vm, vs = v_cache
        self._keep = (params, q, k_cache, v_cache, k_resid, v_resid, table, workspace, out)
        self._s = _shape(q.shape[0], q.shape[1], kc.shape[1], 0, 0, kc.shape[2], k_resid.shape[2],
                         softmax_scale)
        self._args = [ctypes.byref(params.c), ctypes.byref(self._s)]
        self._rope = None
        lib = _lib.load()
        if rope_base is not None:
            self._rope = _lib.nsn_rope(0, float(rope_base))
            self._args.append(ctypes.byref(self._rope))
            self._fn = lib.nsn_decode_attention_rope
        else:
            self._fn = lib.nsn_decode_attention
        self._args += [_ptr(q), _ptr(kc), _ptr(km), _ptr(ks), _ptr(vc), _ptr(vm), _ptr(vs),
                       _ptr(k_resid), _ptr(v_resid), _ptr(table), _ptr(workspace),
                       workspace.numel() * workspace.element_size(), _ptr(out)]

    def __call__(self, n_quant_tok, n_resid_tok, q_pos=None, stream=None):
        self._s.n_quant_tok = n_quant_tok
        self._s.n_resid_tok = n_resid_tok
        if self._rope is not None:
            if q_pos is None:
                raise ValueError("q_pos is required with rotary keys")
            self._rope.q_pos = q_pos
        status = self._fn(*self._args, _stream(stream))
        if status != _lib.NSN_OK:
            _lib.check(status)
