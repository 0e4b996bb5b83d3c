"""The C-ABI library loads, exports every function include/nsn.h declares, and
rejects invalid arguments before any HIP call (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

from kv_cache_calibration_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsn.h")

FAKE = ctypes.c_void_p(0x10000)        # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10004)
NULL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nsn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def P(sub_dim=4, G=128, flags=1, d=128, K=256):
    return ctypes.byref(_lib.nsn_params(d, sub_dim, K, G, flags))


def test_header_declares_the_four_method_calls():
    names = declared_functions()
    for n in ("nsn_build_codebook", "nsn_quantize", "nsn_dequantize", "nsn_decode_attention"):
        assert n in names


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.nsn_version().decode().startswith("nsnq")
    for s in range(6):
        assert lib.nsn_status_string(s) not in (b"", b"unknown status")
    assert lib.nsn_status_string(99) == b"unknown status"


def _q(lib, params, n_seq=2, n_tok=256, x=FAKE, codes=FAKE, meta=FAKE, shift=FAKE,
       xs=None, cs=None, ms=None, ss=None, dtype=0, table=FAKE):
    nsub = 32
    xs = n_tok * 128 if xs is None else xs
    cs = n_tok * nsub if cs is None else cs
    ms = n_tok * 2 if ms is None else ms
    ss = (n_tok // 128) * 128 if ss is None else ss
    return lib.nsn_quantize(params, dtype, x, n_seq, n_tok, xs, table, codes, cs, meta, ms,
                            shift, ss, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(params=None), _lib.NSN_ERR_INVALID_ARG),
    (dict(params=P(d=64)), _lib.NSN_ERR_UNSUPPORTED),
    (dict(params=P(sub_dim=2)), _lib.NSN_ERR_UNSUPPORTED),
    (dict(params=P(K=512)), _lib.NSN_ERR_UNSUPPORTED),
    (dict(params=P(G=64)), _lib.NSN_ERR_UNSUPPORTED),
    (dict(params=P(flags=8)), _lib.NSN_ERR_INVALID_ARG),
    (dict(n_tok=200), _lib.NSN_ERR_INVALID_ARG),
    (dict(n_tok=-128), _lib.NSN_ERR_INVALID_ARG),
    (dict(x=NULL), _lib.NSN_ERR_INVALID_ARG),
    (dict(table=NULL), _lib.NSN_ERR_INVALID_ARG),
    (dict(codes=MISALIGNED), _lib.NSN_ERR_INVALID_ARG),
    (dict(xs=100), _lib.NSN_ERR_INVALID_ARG),
    (dict(cs=8), _lib.NSN_ERR_INVALID_ARG),
    (dict(ms=3), _lib.NSN_ERR_INVALID_ARG),
    (dict(ss=7), _lib.NSN_ERR_INVALID_ARG),
    (dict(dtype=7), _lib.NSN_ERR_INVALID_ARG),
])
def test_quantize_validation(lib, kw, status):
    params = kw.pop("params", P())
    st = _q(lib, params, **kw)
    assert st == status
    assert lib.nsn_last_error()


def test_quantize_empty_is_ok_without_touching_pointers(lib):
    assert _q(lib, P(), n_seq=0, x=NULL, codes=NULL, meta=NULL, shift=NULL) == _lib.NSN_OK
    assert _q(lib, P(), n_tok=0, x=NULL, codes=NULL, meta=NULL, shift=NULL) == _lib.NSN_OK


def test_dequantize_validation(lib):
    f = lib.nsn_dequantize
    ok_args = dict(codes=FAKE, cs=256 * 32, meta=FAKE, ms=512, shift=FAKE, ss=256, table=FAKE,
                   n_seq=2, n_tok=256, dt=0, out=FAKE, os_=256 * 128)

    def call(**kw):
        a = dict(ok_args, **kw)
        return f(P(), a["codes"], a["cs"], a["meta"], a["ms"], a["shift"], a["ss"], a["table"],
                 a["n_seq"], a["n_tok"], a["dt"], a["out"], a["os_"], NULL)
    assert call(n_tok=100) == _lib.NSN_ERR_INVALID_ARG
    assert call(out=NULL) == _lib.NSN_ERR_INVALID_ARG
    assert call(dt=5) == _lib.NSN_ERR_INVALID_ARG
    assert call(os_=64) == _lib.NSN_ERR_INVALID_ARG
    assert call(meta=MISALIGNED) == _lib.NSN_ERR_INVALID_ARG
    assert call(n_seq=0, codes=NULL) == _lib.NSN_OK


def test_build_codebook_validation(lib):
    f = lib.nsn_build_codebook
    ws = lib.nsn_build_codebook_workspace_size(4, 256, 65536)
    assert ws >= 65536 * 4 + 256 * 4 * 8
    assert f(3, 256, 65536, 20, FAKE, FAKE, FAKE, ws, NULL) == _lib.NSN_ERR_UNSUPPORTED
    assert f(4, 128, 65536, 20, FAKE, FAKE, FAKE, ws, NULL) == _lib.NSN_ERR_UNSUPPORTED
    assert f(4, 256, 100, 20, FAKE, FAKE, FAKE, ws, NULL) == _lib.NSN_ERR_INVALID_ARG
    assert f(4, 256, 65536, 0, FAKE, FAKE, FAKE, ws, NULL) == _lib.NSN_ERR_INVALID_ARG
    assert f(4, 256, 65536, 20, NULL, FAKE, FAKE, ws, NULL) == _lib.NSN_ERR_INVALID_ARG
    assert f(4, 256, 65536, 20, FAKE, FAKE, FAKE, ws - 1, NULL) == _lib.NSN_ERR_WORKSPACE


def test_tune_codebook_validation(lib):
    f = lib.nsn_tune_codebook
    ws = lib.nsn_tune_codebook_workspace_size(4, 256, 2048)
    assert ws >= 2048 * 32 * 4 + 2048 * 16 + 3 * 256 * 4 * 8
    assert lib.nsn_tune_codebook_workspace_size(3, 256, 2048) == 0
    assert lib.nsn_tune_codebook_workspace_size(4, 256, 0) == 0
    assert f(3, 256, 2048, 10, 1e-3, FAKE, FAKE, FAKE, ws, NULL) == _lib.NSN_ERR_UNSUPPORTED
    assert f(4, 512, 2048, 10, 1e-3, FAKE, FAKE, FAKE, ws, NULL) == _lib.NSN_ERR_UNSUPPORTED
    assert f(4, 256, 0, 10, 1e-3, FAKE, FAKE, FAKE, ws, NULL) == _lib.NSN_ERR_INVALID_ARG
    assert f(4, 256, (1 << 21) + 1, 10, 1e-3, FAKE, FAKE, FAKE, ws, NULL) == _lib.NSN_ERR_INVALID_ARG
    assert f(4, 256, 2048, -1, 1e-3, FAKE, FAKE, FAKE, ws, NULL) == _lib.NSN_ERR_INVALID_ARG
    for lr in (0.0, -1e-3, 2.0, float("nan"), float("inf")):
        assert f(4, 256, 2048, 10, lr, FAKE, FAKE, FAKE, ws, NULL) == _lib.NSN_ERR_INVALID_ARG
    assert f(4, 256, 2048, 10, 1e-3, NULL, FAKE, FAKE, ws, NULL) == _lib.NSN_ERR_INVALID_ARG
    assert f(4, 256, 2048, 10, 1e-3, FAKE, MISALIGNED, FAKE, ws, NULL) == _lib.NSN_ERR_INVALID_ARG
    assert f(4, 256, 2048, 10, 1e-3, FAKE, FAKE, FAKE, ws - 1, NULL) == _lib.NSN_ERR_WORKSPACE


def test_prepare_and_append_validation(lib):
    ts = lib.nsn_table_size(P())
    assert ts >= 256 * 8 * 4
    assert lib.nsn_prepare_codebook(P(), FAKE, FAKE, ts - 1, NULL) == _lib.NSN_ERR_WORKSPACE
    assert lib.nsn_prepare_codebook(P(), NULL, FAKE, ts, NULL) == _lib.NSN_ERR_INVALID_ARG
    a = lib.nsn_residual_append
    assert a(FAKE, 4, FAKE, 128 * 128, 128, 128, NULL) == _lib.NSN_ERR_INVALID_ARG  # pos == cap
    assert a(FAKE, 4, FAKE, 128 * 128, 128, -1, NULL) == _lib.NSN_ERR_INVALID_ARG
    assert a(FAKE, 4, FAKE, 100, 128, 3, NULL) == _lib.NSN_ERR_INVALID_ARG  # stride too small
    assert a(NULL, 0, NULL, 0, 128, 3, NULL) == _lib.NSN_OK
    # more sequences than one launch's 2^32 work-items cover (16 per sequence)
    assert a(FAKE, 1 << 28, FAKE, 128 * 128, 128, 3, NULL) == _lib.NSN_ERR_UNSUPPORTED


def _shape(**kw):
    d = dict(batch=2, n_q_heads=8, n_kv_heads=2, n_quant_tok=1024, n_resid_tok=16,
             cache_capacity=1024, resid_capacity=128, softmax_scale=0.0884)
    d.update(kw)
    return _lib.nsn_attn_shape(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=6, n_kv_heads=4), _lib.NSN_ERR_INVALID_ARG),
    (dict(n_quant_tok=1000), _lib.NSN_ERR_INVALID_ARG),
    (dict(cache_capacity=512), _lib.NSN_ERR_INVALID_ARG),
    (dict(n_resid_tok=200), _lib.NSN_ERR_INVALID_ARG),
    (dict(n_quant_tok=0, n_resid_tok=0), _lib.NSN_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), _lib.NSN_ERR_INVALID_ARG),
    (dict(batch=0), _lib.NSN_ERR_INVALID_ARG),
    (dict(n_resid_tok=2000, resid_capacity=4096), _lib.NSN_ERR_UNSUPPORTED),
    (dict(batch=65536), _lib.NSN_ERR_UNSUPPORTED),
    # one kv head with 2^18 query heads: 65536 rows of head blocks, one more
    # than a launch's second grid dimension holds
    (dict(n_q_heads=1 << 18, n_kv_heads=1), _lib.NSN_ERR_UNSUPPORTED),
])
def test_attention_validation(lib, kw, status):
    s = _shape(**kw)
    args = [FAKE] * 10
    st = lib.nsn_decode_attention(P(), ctypes.byref(s), *args, FAKE, 1 << 30, FAKE, NULL)
    assert st == status
    assert lib.nsn_decode_attention_workspace_size(P(), ctypes.byref(s)) == 0


def test_attention_workspace_size_and_check(lib):
    s = _shape()
    need = lib.nsn_decode_attention_workspace_size(P(), ctypes.byref(s))
    assert need > 0 and need % 4 == 0
    args = [FAKE] * 10
    st = lib.nsn_decode_attention(P(), ctypes.byref(s), *args, FAKE, need - 4, FAKE, NULL)
    assert st == _lib.NSN_ERR_WORKSPACE
    st = lib.nsn_decode_attention(P(), ctypes.byref(s), *args, NULL, need, FAKE, NULL)
    assert st == _lib.NSN_ERR_INVALID_ARG


def test_attention_workspace_covers_every_fill_level(lib):
    """One size query at a cache's capacity covers every smaller n_quant_tok
    (the split plan rounds chunks to whole groups, so its own count is not
    monotone in the token count); checked on shapes where it was not."""
    for B, Hq, Hkv, G, cap in [(1, 32, 8, 128, 65536), (2, 8, 2, 128, 131072), (1, 4, 1, 256, 32768),
                               (16, 32, 8, 128, 32768), (3, 12, 4, 128, 8192)]:
        def size(n):
            s = _lib.nsn_attn_shape(B, Hq, Hkv, n, 1, cap, 1, 0.088)
            return lib.nsn_decode_attention_workspace_size(P(G=G), ctypes.byref(s))
        sizes = [size(n) for n in range(0, cap + 1, G)]
        assert all(a <= b for a, b in zip(sizes, sizes[1:])), (B, Hq, Hkv, G)
        full = sizes[-1]
        args = [FAKE] * 10
        r = _lib.nsn_rope(10, 10000.0)
        for n in range(G, cap + 1, G):
            # the plan depends on the residual length too (the last chunk is
            # shortened for it); the size query does not, and must cover it
            for nr in (0, 1, 77, 1024):
                s = _lib.nsn_attn_shape(B, Hq, Hkv, n, nr, cap, max(nr, 1), 0.088)
                # one byte short of the query's answer at n: rejected before any
                # launch (a plan above the bound would say NSN_ERR_INTERNAL)
                st = lib.nsn_decode_attention(P(G=G), ctypes.byref(s), *args, FAKE, size(n) - 1, FAKE, NULL)
                assert st == _lib.NSN_ERR_WORKSPACE, (B, Hq, Hkv, G, n, nr, st)
                st = lib.nsn_decode_attention_rope(P(G=G), ctypes.byref(s), ctypes.byref(r), *args, FAKE,
                                                   size(n) - 1, FAKE, NULL)
                assert st == _lib.NSN_ERR_WORKSPACE, (B, Hq, Hkv, G, n, nr, st)
            assert size(n) <= full


@pytest.mark.parametrize("q_pos,base,status", [
    (10, 1.0, _lib.NSN_ERR_INVALID_ARG),            # base must exceed 1
    (10, float("inf"), _lib.NSN_ERR_INVALID_ARG),
    (10, float("nan"), _lib.NSN_ERR_INVALID_ARG),
    (-1, 10000.0, _lib.NSN_ERR_INVALID_ARG),        # negative position
    ((1 << 40) + 1, 10000.0, _lib.NSN_ERR_INVALID_ARG),
])
def test_attention_rope_validation(lib, q_pos, base, status):
    s = _shape()
    r = _lib.nsn_rope(q_pos, base)
    args = [FAKE] * 10
    st = lib.nsn_decode_attention_rope(P(), ctypes.byref(s), ctypes.byref(r), *args, FAKE, 1 << 30,
                                       FAKE, NULL)
    assert st == status
    st = lib.nsn_decode_attention_rope(P(), ctypes.byref(s), None, *args, FAKE, 1 << 30, FAKE, NULL)
    assert st == _lib.NSN_ERR_INVALID_ARG
    # the shape checks are those of nsn_decode_attention
    bad = _shape(n_quant_tok=1000)
    ok = _lib.nsn_rope(10, 10000.0)
    st = lib.nsn_decode_attention_rope(P(), ctypes.byref(bad), ctypes.byref(ok), *args, FAKE,
                                       1 << 30, FAKE, NULL)
    assert st == _lib.NSN_ERR_INVALID_ARG


def test_double_quantization_validation(lib):
    DQ = _lib.NSN_SCALE_ADJUST | _lib.NSN_DQ
    # groups of 128 only, fp16 input only
    assert _q(lib, P(G=256, flags=DQ), ms=256, ss=68) == _lib.NSN_ERR_UNSUPPORTED
    assert _q(lib, P(flags=DQ), ms=256, ss=2 * 68, dtype=1) == _lib.NSN_ERR_UNSUPPORTED
    # meta holds s2' alone and shift the 68-uint16 records: the strides follow
    assert _q(lib, P(flags=DQ), ms=255, ss=2 * 68) == _lib.NSN_ERR_INVALID_ARG
    assert _q(lib, P(flags=DQ), ms=256, ss=2 * 68 - 4) == _lib.NSN_ERR_INVALID_ARG
    assert _q(lib, P(flags=DQ), ms=256, ss=2 * 68 + 2) == _lib.NSN_ERR_INVALID_ARG
    assert _q(lib, P(flags=DQ), n_seq=0, ms=256, ss=2 * 68) == _lib.NSN_OK
    f = lib.nsn_dequantize
    assert f(P(flags=DQ), FAKE, 256 * 32, FAKE, 255, FAKE, 136, FAKE, 2, 256, 0, FAKE, 256 * 128,
             NULL) == _lib.NSN_ERR_INVALID_ARG
    assert f(P(G=256, flags=DQ), FAKE, 256 * 32, FAKE, 256, FAKE, 136, FAKE, 2, 256, 0, FAKE,
             256 * 128, NULL) == _lib.NSN_ERR_UNSUPPORTED
    # group records are 8-byte aligned, so with NSN_DQ the shift pointer needs
    # only 8-byte alignment; 4 is still rejected, and 8 without the flag
    assert _q(lib, P(flags=DQ), ms=256, ss=2 * 68, shift=ctypes.c_void_p(0x10004)) == _lib.NSN_ERR_INVALID_ARG
    assert _q(lib, P(), shift=ctypes.c_void_p(0x10008)) == _lib.NSN_ERR_INVALID_ARG
    # groups of 128 only, with rotary keys too
    s = _shape()
    r = _lib.nsn_rope(10, 10000.0)
    args = [FAKE] * 10
    st = lib.nsn_decode_attention_rope(P(G=256, flags=DQ), ctypes.byref(s), ctypes.byref(r), *args,
                                       FAKE, 1 << 30, FAKE, NULL)
    assert st == _lib.NSN_ERR_UNSUPPORTED
    assert lib.nsn_decode_attention_workspace_size(P(flags=DQ), ctypes.byref(s)) > 0
    assert lib.nsn_decode_attention_workspace_size(P(G=256, flags=DQ), ctypes.byref(s)) == 0


def test_binding_inner_layout_checks():
    torch = pytest.importorskip("torch")
    import kv_cache_calibration_amd as nsnq
    t = torch.zeros((4, 256, 32), dtype=torch.uint8)
    nsnq._inner_contig(t, None)
    nsnq._inner_contig(t[:, 128:], None)          # a group-offset view of a cache
    nsnq._inner_contig(t, (256, 32))
    with pytest.raises(ValueError):
        nsnq._inner_contig(t, (256, 16))
    with pytest.raises(ValueError):
        nsnq._inner_contig(t[:, :, :16], None)     # inner dim not contiguous
    with pytest.raises(ValueError):
        nsnq._dev(t)                              # host tensors are rejected
    p = nsnq.Params(sub_dim=8, group_size=256, scale_adjust=False)
    assert (p.c.sub_dim, p.c.group_size, p.c.flags, p.c.head_dim) == (8, 256, 0, 128)


def test_binding_layout_checks_of_both_metadata_layouts():
    """The binding checks meta / shift / cache shapes against the layout the
    params select, before any call (host tensors suffice here)."""
    torch = pytest.importorskip("torch")
    import kv_cache_calibration_amd as nsnq
    p = nsnq.Params(sub_dim=4, group_size=128)
    pd = nsnq.Params(sub_dim=4, group_size=128, dq=True)
    assert pd.dq and not p.dq and pd.c.flags == _lib.NSN_SCALE_ADJUST | _lib.NSN_DQ
    meta = torch.zeros((2, 256, 2), dtype=torch.float16)
    shift = torch.zeros((2, 2, 128), dtype=torch.float16)
    meta_dq = torch.zeros((2, 256), dtype=torch.float16)
    recs = torch.zeros((2, 2, 136), dtype=torch.uint8)
    nsnq._check_meta_layout(p, meta, shift)
    nsnq._check_meta_layout(pd, meta_dq, recs)
    nsnq._check_meta_layout(pd, meta_dq, recs.view(torch.int16))
    for args in ((p, meta_dq, recs), (pd, meta, shift), (pd, meta_dq, recs[:, :, :135])):
        with pytest.raises(ValueError):
            nsnq._check_meta_layout(*args)
    with pytest.raises(ValueError):
        nsnq._stride16(torch.zeros((3, 135), dtype=torch.uint8))
    assert nsnq._stride16(recs) == 136
    # attention shapes
    B, Hq, Hkv, cap, R = 2, 8, 2, 256, 16
    q = torch.zeros((B, Hq, 128), dtype=torch.float16)
    out = torch.zeros((B, Hq, 128), dtype=torch.float32)
    kc = torch.zeros((B, Hkv, cap, 32), dtype=torch.uint8)
    plain = (kc, torch.zeros((B, Hkv, cap, 2), dtype=torch.float16),
             torch.zeros((B, Hkv, cap // 128, 128), dtype=torch.float16))
    dq = (kc, torch.zeros((B, Hkv, cap), dtype=torch.float16),
          torch.zeros((B, Hkv, cap // 128, 136), dtype=torch.uint8))
    kr = torch.zeros((B, Hkv, R, 128), dtype=torch.float16)
    nsnq._check_attention_shapes(p, q, plain, plain, kr, kr, out)
    nsnq._check_attention_shapes(pd, q, dq, dq, kr, kr, out)
    with pytest.raises(ValueError):
        nsnq._check_attention_shapes(p, q, dq, dq, kr, kr, out)
    with pytest.raises(ValueError):
        nsnq._check_attention_shapes(pd, q, plain, plain, kr, kr, out)
    with pytest.raises(ValueError):
        nsnq._check_attention_shapes(p, q, plain, plain, kr, kr[:, :, :8], out)
    with pytest.raises(ValueError):
        nsnq._check_attention_shapes(nsnq.Params(sub_dim=8), q, plain, plain, kr, kr, out)


def test_cache_layout_helper():
    torch = pytest.importorskip("torch")
    import kv_cache_calibration_amd as nsnq
    c, m, s = nsnq.cache_layout(nsnq.Params(sub_dim=4), 3, 256)
    assert c == ((3, 256, 32), torch.uint8) and m == ((3, 256, 2), torch.float16)
    assert s == ((3, 2, 128), torch.float16)
    c, m, s = nsnq.cache_layout(nsnq.Params(sub_dim=8, dq=True), 3, 256)
    assert c == ((3, 256, 16), torch.uint8) and m == ((3, 256), torch.float16)
    assert s == ((3, 2, 136), torch.uint8)
    meta = torch.zeros(m[0], dtype=m[1])
    shift = torch.zeros(s[0], dtype=s[1])
    nsnq._check_meta_layout(nsnq.Params(sub_dim=8, dq=True), meta, shift)
    with pytest.raises(ValueError):
        nsnq.cache_layout(nsnq.Params(), 1, 100)


def test_binding_rejects_wrong_dtypes_and_sizes():
    """The binding checks what the C ABI cannot see: dtypes, the table size
    and token counts (host tensors suffice; the checks run before any call)."""
    torch = pytest.importorskip("torch")
    import kv_cache_calibration_amd as nsnq
    p = nsnq.Params(sub_dim=4)
    with pytest.raises(ValueError):
        nsnq._check_codes(p, torch.zeros((2, 256, 16), dtype=torch.uint8))   # 1-bit width for 2-bit params
    with pytest.raises(ValueError):
        nsnq._check_codes(p, torch.zeros((2, 256, 32), dtype=torch.int16))
    nsnq._check_codes(p, torch.zeros((2, 256, 32), dtype=torch.uint8))
    B, Hq, Hkv, cap, R = 1, 4, 1, 128, 4
    kc = torch.zeros((B, Hkv, cap, 32), dtype=torch.uint8)
    plain = (kc, torch.zeros((B, Hkv, cap, 2), dtype=torch.float16),
             torch.zeros((B, Hkv, 1, 128), dtype=torch.float16))
    kr = torch.zeros((B, Hkv, R, 128), dtype=torch.float16)
    q = torch.zeros((B, Hq, 128), dtype=torch.float16)
    out = torch.zeros((B, Hq, 128), dtype=torch.float32)
    nsnq._check_attention_shapes(p, q, plain, plain, kr, kr, out)
    with pytest.raises(ValueError):
        nsnq._check_attention_shapes(p, q.float(), plain, plain, kr, kr, out)
    with pytest.raises(ValueError):
        nsnq._check_attention_shapes(p, q, plain, plain, kr, kr, out.half())
    with pytest.raises(ValueError):
        nsnq._check_attention_shapes(p, q, plain, plain, kr.float(), kr, out)


def test_prepared_attention_checks_its_tensors_once():
    """PreparedDecodeAttention runs the per-call function's checks at
    construction: host tensors, a wrong dtype or a short table are refused
    before anything is marshalled (no GPU needed)."""
    torch = pytest.importorskip("torch")
    import kv_cache_calibration_amd as nsnq
    p = nsnq.Params(sub_dim=4)
    B, Hq, Hkv, cap, R = 1, 4, 1, 128, 4
    kc = torch.zeros((B, Hkv, cap, 32), dtype=torch.uint8)
    plain = (kc, torch.zeros((B, Hkv, cap, 2), dtype=torch.float16),
             torch.zeros((B, Hkv, 1, 128), dtype=torch.float16))
    kr = torch.zeros((B, Hkv, R, 128), dtype=torch.float16)
    q = torch.zeros((B, Hq, 128), dtype=torch.float16)
    out = torch.zeros((B, Hq, 128), dtype=torch.float32)
    table = torch.zeros(16, dtype=torch.uint8)
    work = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="device"):
        nsnq.PreparedDecodeAttention(p, q, plain, plain, kr, kr, table, work, out, 0.1)
    with pytest.raises(ValueError):
        nsnq._check_attention_call(p, q.float(), plain, plain, kr, kr, table, work, out)


def test_binding_refuses_a_table_prepared_for_other_params():
    """A table tensor prepared through the binding carries the (sub_dim, dq)
    it was made for; calls with other params are refused, an untagged table
    is checked for its size only (host tensors, no GPU needed)."""
    torch = pytest.importorskip("torch")
    import kv_cache_calibration_amd as nsnq
    p4, p8, p4dq = nsnq.Params(sub_dim=4), nsnq.Params(sub_dim=8), nsnq.Params(sub_dim=4, dq=True)
    table = torch.zeros(nsnq.nsn_table_size(p4), dtype=torch.uint8)
    for p in (p4, p8, p4dq):
        nsnq._check_table(p, table)
    table._nsn_prepared_for = nsnq._table_key(p4)
    nsnq._check_table(p4, table)
    nsnq._check_table(nsnq.Params(sub_dim=4, group_size=256, scale_adjust=False), table)
    for p in (p8, p4dq):
        with pytest.raises(ValueError, match="prepared for"):
            nsnq._check_table(p, table)


def test_prepared_append_checks_its_tensors_once():
    """PreparedResidualAppend runs the per-call function's checks at
    construction: host tensors are refused before anything is marshalled."""
    torch = pytest.importorskip("torch")
    import kv_cache_calibration_amd as nsnq
    tok = torch.zeros((4, 128), dtype=torch.float16)
    resid = torch.zeros((4, 16, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="device"):
        nsnq.PreparedResidualAppend(tok, resid)


def test_binding_checks_sequence_and_group_extents():
    """The C ABI trusts the sequence count and the group slots it is given:
    the binding rejects codes, meta or shift tensors with fewer sequences
    than the input, a shift view ending before the last group, and a
    non-fp16 meta or shift (host tensors; the checks run before any call)."""
    torch = pytest.importorskip("torch")
    import kv_cache_calibration_amd as nsnq
    p = nsnq.Params(sub_dim=4, group_size=128)
    n_seq, T = 3, 512
    codes = torch.zeros((n_seq, T, 32), dtype=torch.uint8)
    meta = torch.zeros((n_seq, T, 2), dtype=torch.float16)
    shift = torch.zeros((n_seq, T // 128, 128), dtype=torch.float16)
    nsnq._check_extents(p, n_seq, T, codes, meta, shift)
    nsnq._check_extents(p, n_seq, T - 128, codes, meta, shift[:, :3])
    for args in ((codes[:2], meta, shift), (codes, meta[:2], shift), (codes, meta, shift[:1]),
                 (codes, meta, shift[:, :3]), (codes[:, :384], meta, shift), (codes, meta[:, :500], shift)):
        with pytest.raises(ValueError):
            nsnq._check_extents(p, n_seq, T, *args)
    with pytest.raises(ValueError):
        nsnq._check_meta_layout(p, meta.view(torch.int16), shift)
    with pytest.raises(ValueError):
        nsnq._check_meta_layout(p, meta, shift.view(torch.bfloat16))


def test_launch_size_limits_are_rejected_up_front(lib):
    """A call whose single launch would need 2^32 or more work-items is
    refused with NSN_ERR_UNSUPPORTED before any HIP call (fake pointers,
    nothing launched); one group below the limit passes validation (checked
    on the error path only: a too-small stride makes it fail afterwards)."""
    G = 128
    limit = (1 << 24) - 1
    # n_seq = 1: no strides checked, so the group count decides
    st = _q(lib, P(), n_seq=1, n_tok=(limit + 1) * G, xs=0, cs=0, ms=0, ss=0)
    assert st == _lib.NSN_ERR_UNSUPPORTED
    assert b"token groups" in lib.nsn_last_error()
    st = lib.nsn_dequantize(P(), FAKE, 0, FAKE, 0, FAKE, 0, FAKE, 1, (limit + 1) * G, 0, FAKE, 0, NULL)
    assert st == _lib.NSN_ERR_UNSUPPORTED
    # strides are checked before the count: a short stride still reports
    # INVALID_ARG at a count within the limit (nothing is launched)
    st = _q(lib, P(), n_seq=2, n_tok=(limit // 2) * G, xs=100)
    assert st == _lib.NSN_ERR_INVALID_ARG
    st = lib.nsn_nearest_codeword(P(), FAKE, FAKE, (1 << 32) - 255, FAKE, NULL)
    assert st == _lib.NSN_ERR_UNSUPPORTED


def _no_hip_device():
    torch = pytest.importorskip("torch")
    return torch.cuda.device_count() == 0


def test_failed_launch_reports_nsn_err_hip(lib):
    """A launch that the HIP runtime refuses comes back as NSN_ERR_HIP with
    the runtime's message.  Forced from the host: with no HIP device visible
    every launch fails, so valid arguments (fake device pointers, never
    dereferenced) reach the launch and fail there.  Skipped where a device
    exists, since there the launch would run on the fake pointers."""
    if not _no_hip_device():
        pytest.skip("a HIP device is visible: a launch on fake pointers would run")
    st = _q(lib, P(), n_seq=1, n_tok=128, xs=0, cs=0, ms=0, ss=0)
    assert st == _lib.NSN_ERR_HIP
    msg = lib.nsn_last_error().decode()
    assert msg.startswith("nsn_quantize launch:") and len(msg) > len("nsn_quantize launch: ")
    st = lib.nsn_residual_append(FAKE, 1, FAKE, 0, 4, 0, NULL)
    assert st == _lib.NSN_ERR_HIP
    # a later successful call clears the detail string
    assert _q(lib, P(), n_seq=0) == _lib.NSN_OK
    assert lib.nsn_last_error() == b""


def test_randomized_rotation_flag(lib):
    """NSN_RHT is a known flag; the rotary attention call refuses it before
    touching any pointer; the binding packs +-1 signs into the bit mask
    (bit c of word c / 32 for a negated channel c)."""
    import kv_cache_calibration_amd as nsnq
    RHT = _lib.NSN_SCALE_ADJUST | _lib.NSN_RHT
    assert lib.nsn_table_size(P(flags=RHT)) > 0
    assert lib.nsn_table_size(P(flags=RHT | 8)) == 0
    s = _shape()
    r = _lib.nsn_rope(10, 10000.0)
    args = [FAKE] * 10
    st = lib.nsn_decode_attention_rope(P(flags=RHT), ctypes.byref(s), ctypes.byref(r), *args, FAKE,
                                       1 << 30, FAKE, NULL)
    assert st == _lib.NSN_ERR_UNSUPPORTED
    assert b"NSN_RHT" in lib.nsn_last_error()
    signs = [1.0] * 128
    for c in (0, 31, 32, 77, 127):
        signs[c] = -1.0
    p = nsnq.Params(rht_signs=signs)
    assert p.rht and p.c.flags == RHT
    assert list(p.c.rht_signs) == [(1 << 0) | (1 << 31), 1 << 0, 1 << 13, 1 << 31]
    assert not nsnq.Params().rht and list(nsnq.Params().c.rht_signs) == [0, 0, 0, 0]
    with pytest.raises(ValueError):
        nsnq.Params(rht_signs=[1.0] * 127)
    with pytest.raises(ValueError):
        nsnq.Params(rht_signs=[0.0] * 128)
