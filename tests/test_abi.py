"""C-ABI contract tests that need no GPU: symbols, layout arithmetic and every
error path (all argument checks run before the first HIP call)."""
import ctypes as C
import os
import re

import pytest

import bit_linear_amd as dv
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dvssq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dvssq_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(dv.EXPORTS)
    lib = C.CDLL(dv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_library_exports_nothing_else():
    """Internal host symbols are hidden: the text symbols of the dynamic symbol
    table are exactly the declared entry points."""
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", dv.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    text = {ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3 and ln.split()[1] in "TW"}
    assert text == set(declared_functions())


def test_layout_struct_size_matches_header():
    # 10 int32 + 10 int64 fields, no padding
    assert C.sizeof(dv.Layout) == 10 * 4 + 10 * 8


@pytest.mark.parametrize("N,K,r,block,n_seg", [
    (512, 256, 4, 256, 1), (10240, 2560, 16, 256, 1), (2560, 10240, 16, 256, 1),
    (20480, 2560, 24, 256, 2), (6144, 2048, 16, 2048, 1), (2048, 6144, 32, 2048, 1),
    (520, 192, 1, 64, 1), (48, 128, 64, 128, 1),
])
def test_pack_info_matches_oracle_layout(N, K, r, block, n_seg):
    L = dv.pack_info(N, K, r, block, n_seg, M_max=4096)
    ref = oracle.layout(N, K, r, n_seg)
    assert L.n_int4 == ref["N4"] and L.n_int8 == ref["N8"]
    for k in ("off_idx", "off_q4", "off_s4", "off_q8", "off_s8", "off_U", "off_V",
              "blob_bytes", "algo_bytes"):
        assert getattr(L, k) == ref[k], k
    assert (L.N, L.K, L.r, L.block, L.group, L.n_seg, L.M_max) == (N, K, r, block, 64, n_seg, 4096)
    assert L.ws_bytes > 0 and L.ws_bytes % 256 == 0


def test_algo_bytes_of_workloads():
    # packed sizes of the benchmark layers (bytes of the layer itself, no padding)
    assert dv.pack_info(512, 256, 4, 256).algo_bytes == 85_760
    assert dv.pack_info(10240, 2560, 16, 256).algo_bytes == 15_918_080
    assert dv.pack_info(2560, 10240, 16, 256).algo_bytes == 15_883_520
    assert dv.pack_info(20480, 2560, 24, 256, 2).algo_bytes == 32_245_760
    assert dv.pack_info(6144, 2048, 16, 2048).algo_bytes == 7_711_744
    assert dv.pack_info(2048, 6144, 16, 2048).algo_bytes == 7_693_312


def rc_pack(*args):
    out = dv.Layout()
    return dv.lib().dvssq_pack_info(*args, C.byref(out))


@pytest.mark.parametrize("args,code", [
    ((512, 256, 4, 256, 1, 32), dv.DVSSQ_OK),
    ((0, 256, 4, 256, 1, 32), dv.DVSSQ_EINVAL),        # N <= 0
    ((516, 256, 4, 256, 1, 32), dv.DVSSQ_EINVAL),      # N % 8
    ((520, 256, 4, 256, 2, 32), dv.DVSSQ_EINVAL),      # N % 16 with two segments
    ((512, 200, 4, 256, 1, 32), dv.DVSSQ_EINVAL),      # K % 64
    ((512, 320, 4, 256, 1, 32), dv.DVSSQ_EINVAL),      # K % block
    ((512, 256, 0, 256, 1, 32), dv.DVSSQ_EINVAL),      # r < 1
    ((512, 256, 65, 256, 1, 32), dv.DVSSQ_EINVAL),     # r > 64
    ((512, 256, 33, 256, 2, 32), dv.DVSSQ_EINVAL),     # n_seg * r > 64
    ((512, 256, 4, 256, 3, 32), dv.DVSSQ_EINVAL),      # n_seg
    ((512, 256, 4, 256, 1, 0), dv.DVSSQ_EINVAL),       # M_max
    ((512, 256, 4, 32, 1, 32), dv.DVSSQ_EUNSUPPORTED),   # block below 64
    ((512, 8192, 4, 4096, 1, 32), dv.DVSSQ_EUNSUPPORTED),  # block above 2048
    ((512, 384, 4, 192, 1, 32), dv.DVSSQ_EUNSUPPORTED),    # not a power of two
])
def test_pack_info_errors(args, code):
    assert rc_pack(*args) == code


def test_pack_info_null_out():
    assert dv.lib().dvssq_pack_info(512, 256, 4, 256, 1, 32, None) == dv.DVSSQ_EINVAL


# Fake, never-dereferenced device addresses: every call below fails validation
# before any HIP call, so they run without a GPU.
BLOB, X, Y, WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def call(fn, L, blob=BLOB, x=X, y=Y, M=1, ws=WS, flags=0):
    f = getattr(dv.lib(), fn)
    return f(C.byref(L) if L is not None else None, blob, x, y, M, ws, flags, None)


@pytest.mark.parametrize("fn", ["dvssq_linear_decode", "dvssq_linear_prefill"])
def test_linear_error_paths(fn):
    L = dv.pack_info(512, 256, 4, 256, 1, M_max=64)
    E = dv.DVSSQ_EINVAL
    assert call(fn, None) == E
    assert call(fn, L, blob=None) == E
    assert call(fn, L, x=None) == E
    assert call(fn, L, y=None) == E
    assert call(fn, L, ws=None) == E
    assert call(fn, L, M=0) == E
    assert call(fn, L, M=65) == E                         # above M_max
    assert call(fn, L, blob=BLOB + 16) == E               # blob not 256-aligned
    assert call(fn, L, ws=WS + 128) == E                  # ws not 256-aligned
    assert call(fn, L, x=X + 2) == E                      # x not 16-aligned
    assert call(fn, L, y=Y + 8) == E                      # y not 16-aligned
    assert call(fn, L, y=X + 256) == E                    # y overlaps x
    assert call(fn, L, y=WS + 1024) == E                  # y overlaps ws
    assert call(fn, L, flags=2) == E                      # unknown flag
    bad = dv.pack_info(512, 256, 4, 256, 1, M_max=64)
    bad.off_V += 256                                      # edited layout
    assert call(fn, bad) == E
    bad2 = dv.pack_info(512, 256, 4, 256, 1, M_max=64)
    bad2.K = 300
    assert call(fn, bad2) == E


def test_decode_rejects_large_m():
    L = dv.pack_info(512, 256, 4, 256, 1, M_max=64)
    assert call("dvssq_linear_decode", L, M=33) == dv.DVSSQ_EUNSUPPORTED


def test_test_only_flag_is_decode_only():
    # DVSSQ_TEST_NO_PUBLISH is a decode flag; the prefill refuses it before any HIP call
    L = dv.pack_info(512, 256, 4, 256, 1, M_max=64)
    assert call("dvssq_linear_prefill", L, M=40, flags=dv.DVSSQ_TEST_NO_PUBLISH) == dv.DVSSQ_EINVAL
    assert call("dvssq_linear_decode", L, M=1, flags=dv.DVSSQ_TEST_NO_PUBLISH | 4) == dv.DVSSQ_EINVAL


def test_workspace_keeps_its_status_area():
    # the first DVSSQ_WS_STATUS_BYTES of a workspace are the status area, never
    # part of the decode or prefill regions: ws_bytes covers it as well
    for args in ((512, 256, 4, 256, 1, 1), (10240, 2560, 16, 256, 1, 32), (6144, 2048, 16, 2048, 1, 4096)):
        L = dv.pack_info(*args)
        assert L.ws_bytes > dv.DVSSQ_WS_STATUS_BYTES and L.ws_bytes % 256 == 0


def test_fwht_error_paths():
    f = dv.lib().dvssq_fwht
    assert f(None, Y, 4, 256, 256, None) == dv.DVSSQ_EINVAL
    assert f(X, None, 4, 256, 256, None) == dv.DVSSQ_EINVAL
    assert f(X, Y, -1, 256, 256, None) == dv.DVSSQ_EINVAL
    assert f(X, Y, 4, 320, 256, None) == dv.DVSSQ_EINVAL       # K % block
    assert f(X, Y, 4, 256, 32, None) == dv.DVSSQ_EUNSUPPORTED
    assert f(X, Y, 4, 96 * 4, 96, None) == dv.DVSSQ_EUNSUPPORTED
    assert f(X + 2, Y, 4, 256, 256, None) == dv.DVSSQ_EINVAL
    assert f(X, X + 512, 4, 256, 256, None) == dv.DVSSQ_EINVAL  # partial overlap
    assert f(X, Y, 0, 256, 256, None) == dv.DVSSQ_OK            # M = 0: nothing to do


def test_status_strings():
    for code in (0, -1, -2, -3, 7, dv.DVSSQ_STATUS_WAIT_TIMEOUT):
        assert isinstance(dv.status_str(code), str) and dv.status_str(code)
    assert dv.status_str(dv.DVSSQ_EINVAL) != dv.status_str(dv.DVSSQ_EHIP)


def test_binding_raises_on_error():
    with pytest.raises(dv.DvssqError) as ei:
        dv.pack_info(516, 256, 4, 256)
    assert ei.value.code == dv.DVSSQ_EINVAL


# ------------------------------------------------------------------ gated MLP block

def test_mlp_ws_bytes_and_pairing():
    gu = dv.pack_info(20480, 2560, 24, 256, 2, M_max=32)
    dn = dv.pack_info(2560, 10240, 16, 256, 1, M_max=32)
    n = dv.mlp_ws_bytes(gu, dn)
    assert n % 256 == 0 and n >= max(gu.ws_bytes, dn.ws_bytes) + 2 * 32 * (20480 + 10240)
    f, out, E = dv.lib().dvssq_mlp_ws_bytes, C.c_int64(0), dv.DVSSQ_EINVAL
    assert f(C.byref(dn), C.byref(gu), C.byref(out)) == E          # swapped pair
    assert f(C.byref(gu), C.byref(dn), None) == E
    assert f(None, C.byref(dn), C.byref(out)) == E
    one = dv.pack_info(20480, 2560, 24, 256, 1, M_max=32)            # not a two-segment layer
    assert f(C.byref(one), C.byref(dn), C.byref(out)) == E
    wrong = dv.pack_info(2560, 5120, 16, 256, 1, M_max=32)           # down K != I
    assert f(C.byref(gu), C.byref(wrong), C.byref(out)) == E


def test_mlp_decode_error_paths():
    gu = dv.pack_info(512, 256, 4, 256, 2, M_max=64)
    dn = dv.pack_info(256, 256, 4, 256, 1, M_max=64)
    GB, DB = 0x10000000, 0x18000000
    f, E = dv.lib().dvssq_mlp_decode, dv.DVSSQ_EINVAL

    def c(g=gu, gb=GB, d=dn, db=DB, x=X, y=Y, M=1, ws=WS, flags=0):
        return f(C.byref(g) if g is not None else None, gb, C.byref(d) if d is not None else None, db, x, y, M,
                 ws, flags, None)

    assert c(g=None) == E and c(d=None) == E
    assert c(gb=None) == E and c(db=None) == E
    assert c(x=None) == E and c(y=None) == E and c(ws=None) == E
    assert c(M=0) == E and c(M=65) == E
    assert c(M=33) == dv.DVSSQ_EUNSUPPORTED
    assert c(flags=2) == E
    assert c(ws=WS + 128) == E and c(x=X + 2) == E and c(y=Y + 8) == E
    assert c(y=X + 256) == E                                   # y overlaps x
    assert c(y=WS + 1024) == E                                 # y overlaps ws
    assert c(g=dn, d=gu) == E                                  # swapped pair
    assert c(flags=dv.DVSSQ_TEST_NO_PUBLISH) == E              # test flag of the layer call only


def test_mlp_prefill_error_paths():
    gu = dv.pack_info(512, 256, 4, 256, 2, M_max=64)
    dn = dv.pack_info(256, 256, 4, 256, 1, M_max=64)
    f, E = dv.lib().dvssq_mlp_prefill, dv.DVSSQ_EINVAL
    GB, DB = 0x10000000, 0x18000000
    assert f(C.byref(gu), None, C.byref(dn), DB, X, Y, 40, WS, 0, None) == E
    assert f(C.byref(gu), GB, C.byref(dn), DB, X, Y, 65, WS, 0, None) == E      # above M_max
    assert f(C.byref(gu), GB, C.byref(dn), DB, X, Y, 0, WS, 0, None) == E
    assert f(C.byref(dn), GB, C.byref(gu), DB, X, Y, 40, WS, 0, None) == E      # swapped pair
    assert f(C.byref(gu), GB + 64, C.byref(dn), DB, X, Y, 40, WS, 0, None) == E  # blob alignment
    assert f(C.byref(gu), GB, C.byref(dn), DB, X, WS + 4096, 40, WS, 0, None) == E  # y inside ws


def test_materialize_error_paths():
    L = dv.pack_info(512, 256, 4, 256, 1, M_max=8)
    f, E = dv.lib().dvssq_materialize, dv.DVSSQ_EINVAL
    assert f(None, BLOB, Y, None) == E
    assert f(C.byref(L), None, Y, None) == E
    assert f(C.byref(L), BLOB, None, None) == E
    assert f(C.byref(L), BLOB + 16, Y, None) == E        # blob not 256-aligned
    assert f(C.byref(L), BLOB, Y + 2, None) == E         # w not 16-aligned
    assert f(C.byref(L), BLOB, BLOB + 4096, None) == E   # w overlaps the blob
    bad = dv.pack_info(512, 256, 4, 256, 1, M_max=8)
    bad.off_U += 256
    assert f(C.byref(bad), BLOB, Y, None) == E


def test_stream_read_error_paths():
    f, E = dv.lib().dvssq_stream_read, dv.DVSSQ_EINVAL
    assert f(None, 1024, Y, None) == E
    assert f(X, 1024, None, None) == E
    assert f(X, 0, Y, None) == E and f(X, 1000, Y, None) == E     # size: positive multiple of 16
    assert f(X + 8, 1024, Y, None) == E                           # buffer alignment
    assert f(X, 1 << 41, Y, None) == E


def test_decode_noalloc_error_paths():
    """The no-allocation decode checks its arguments like dvssq_linear_decode
    (there is no workspace argument), all before any HIP launch."""
    f = dv.lib().dvssq_linear_decode_noalloc
    L = dv.pack_info(512, 256, 4, 256, 1, M_max=64)
    E = dv.DVSSQ_EINVAL

    def c(L=L, blob=BLOB, x=X, y=Y, M=1, flags=0):
        return f(C.byref(L) if L is not None else None, blob, x, y, M, flags, None)

    assert c(L=None) == E and c(blob=None) == E and c(x=None) == E and c(y=None) == E
    assert c(M=0) == E and c(M=65) == E
    assert c(M=33) == dv.DVSSQ_EUNSUPPORTED
    assert c(flags=2) == E
    assert c(blob=BLOB + 16) == E and c(x=X + 2) == E and c(y=Y + 8) == E
    assert c(y=X + 256) == E                                   # y overlaps x
    bad = dv.pack_info(512, 256, 4, 256, 1, M_max=64)
    bad.off_U += 256
    assert c(L=bad) == E


def test_quantize_ws_bytes():
    L = dv.pack_info(512, 256, 4, 256, 1)
    f = dv.lib().dvssq_quantize_ws_bytes
    n = f(C.byref(L), 12)
    # R [N][K], Q [N][l], three [K][l] and the small arrays, each 256-aligned
    assert n >= 8 * (512 * 256 + 512 * 12 + 3 * 256 * 12) and n % 256 == 0
    assert f(C.byref(L), 3) == -1                 # l < r
    assert f(C.byref(L), 257) == -1               # l > min(N / n_seg, K)
    assert f(None, 12) == -1
    seg = dv.pack_info(2 * 256, 256, 4, 256, 2)
    assert f(C.byref(seg), 256) > 0 and f(C.byref(seg), 257) == -1
    with pytest.raises(dv.DvssqError):
        dv.quantize_ws_bytes(L, 2)


def test_quantize_error_paths():
    """Every argument check of the GPU quantizer runs before its first launch."""
    f, E = dv.lib().dvssq_quantize, dv.DVSSQ_EINVAL
    L = dv.pack_info(512, 256, 4, 256, 1)
    OM = 0x50000000

    def c(L=L, W=X, om=OM, l=12, p=2, blob=BLOB, ws=WS):
        return f(C.byref(L) if L is not None else None, W, om, l, p, blob, ws, None)

    assert c(L=None) == E and c(W=None) == E and c(om=None) == E and c(blob=None) == E and c(ws=None) == E
    assert c(l=3) == E and c(l=257) == E
    assert c(p=-1) == E and c(p=17) == E
    assert c(W=X + 8) == E and c(om=OM + 4) == E and c(blob=BLOB + 16) == E and c(ws=WS + 128) == E
    assert c(blob=X + 1024) == E                        # blob inside W
    assert c(ws=BLOB + 256) == E                        # ws inside the blob
    assert c(om=WS + 256) == E                          # sketch inside ws
    bad = dv.pack_info(512, 256, 4, 256, 1)
    bad.off_U += 256
    assert c(L=bad) == E
    # one rotation row (fp64 + codes) must fit the 160 KB of LDS
    big = dv.pack_info(512, 16384, 4, 256, 1)
    assert c(L=big) == dv.DVSSQ_EUNSUPPORTED


def test_kvbss_attention_error_paths():
    """Every argument check of the attention call runs before its launch."""
    f, E = dv.lib().dvssq_kvbss_attention, dv.DVSSQ_EINVAL
    O = 0x60000000

    def shape(**kw):
        d = dict(B=1, Mq=4, Nk=64, Hq=16, Hkv=4, D=256, window=0, scale=0.06875, haze=12.0)
        d.update(kw)
        return dv.AttnShape(**d)

    def c(sh=None, q=X, k=BLOB, v=WS, o=O, ws=None):
        return f(C.byref(sh if sh is not None else shape()), q, k, v, o, ws, None)

    assert f(None, X, BLOB, WS, O, None, None) == E
    assert c(q=None) == E and c(k=None) == E and c(v=None) == E and c(o=None) == E
    assert c(shape(Mq=65)) == E                    # more queries than keys
    assert c(shape(Mq=0)) == E and c(shape(B=0)) == E
    assert c(shape(Hq=6)) == E                     # not a multiple of Hkv
    assert c(shape(window=-1)) == E
    assert c(shape(scale=float("inf"))) == E and c(shape(haze=float("nan"))) == E and c(shape(haze=-1.0)) == E
    assert c(q=X + 8) == E and c(o=O + 2) == E
    assert c(o=X + 64) == E                        # output overlaps q
    assert c(shape(D=96)) == dv.DVSSQ_EUNSUPPORTED
    assert c(shape(B=1, Nk=1 << 20, Hkv=4, D=256)) == dv.DVSSQ_EUNSUPPORTED
    # a decode step over 4096 keys takes the two-launch form: it needs a workspace
    WSA = 0x70000000
    dec = shape(Mq=1, Nk=4096)
    assert c(dec) == E and c(dec, ws=WSA + 64) == E                  # missing / misaligned
    assert c(dec, ws=X) == E                                          # workspace overlaps q


def test_kvbss_attention_ws_bytes():
    f = dv.lib().dvssq_kvbss_attention_ws_bytes
    n = C.c_int64(-1)

    def shape(**kw):
        d = dict(B=1, Mq=1, Nk=32768, Hq=16, Hkv=4, D=256, window=0, scale=0.06875, haze=12.0)
        d.update(kw)
        return dv.AttnShape(**d)

    assert f(C.byref(shape()), C.byref(n)) == dv.DVSSQ_OK
    # logits [4][16][32768] fp32 + range maxima, sums and counters: 64 ranges of 512 keys
    assert n.value >= 4 * 16 * 32768 * 4 + 4 * 64 * 16 * 256 * 4 and n.value % 256 == 0
    assert f(C.byref(shape(Mq=2048, Nk=2048)), C.byref(n)) == dv.DVSSQ_OK and n.value == 0   # one launch
    assert f(C.byref(shape(Nk=512)), C.byref(n)) == dv.DVSSQ_OK and n.value == 0             # one range
    assert f(C.byref(shape(Mq=5, Nk=4096)), C.byref(n)) == dv.DVSSQ_OK and n.value == 0      # 20 rows
    assert f(C.byref(shape()), None) == dv.DVSSQ_EINVAL
    assert f(None, C.byref(n)) == dv.DVSSQ_EINVAL
    assert f(C.byref(shape(D=96)), C.byref(n)) == dv.DVSSQ_EUNSUPPORTED
