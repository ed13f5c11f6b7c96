"""The C-ABI library on the CPU: it loads, exports every symbol include/pkv.h declares, and
rejects invalid arguments on the host before anything is enqueued (no GPU needed: every
call here fails validation, so no HIP runtime call is made)."""
import ctypes
import os
import re

import pytest

from paged_kv_scaled_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x1000)     # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    return B.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for name in ("pkv_kv_cache_write", "pkv_paged_attention_decode", "pkv_paged_attention_prefill",
                 "pkv_kv_cache_gather", "pkv_decode_workspace_size", "pkv_last_error"):
        assert name in syms


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(B.SIGNATURES)


def test_version(lib):
    assert lib.pkv_version() >> 16 == 1


def _write(lib, **kw):
    a = dict(key=FAKE, value=FAKE, stride=256, slots=FAKE, T=4, kc=FAKE, vc=FAKE, bstride=16 * 256,
             nb=8, bs=16, hkv=2, d=128, dt=B.PKV_BF16)
    a.update(kw)
    return lib.pkv_kv_cache_write(a["key"], a["value"], a["stride"], a["slots"], a["T"], a["kc"],
                                  a["vc"], a["bstride"], a["nb"], a["bs"], a["hkv"], a["d"],
                                  a["dt"], NULL)


def test_write_rejections(lib):
    assert _write(lib, key=NULL) == B.PKV_ERR_INVALID_ARG
    assert "NULL" in B.last_error()
    assert _write(lib, kc=NULL) == B.PKV_ERR_INVALID_ARG
    assert _write(lib, bs=12) == B.PKV_ERR_INVALID_ARG
    assert "power of two" in B.last_error()
    assert _write(lib, bs=512, bstride=512 * 256) == B.PKV_ERR_INVALID_ARG
    assert _write(lib, d=96, stride=192, bstride=16 * 192) == B.PKV_ERR_UNSUPPORTED
    assert _write(lib, dt=7) == B.PKV_ERR_UNSUPPORTED
    assert _write(lib, stride=100) == B.PKV_ERR_INVALID_ARG
    assert _write(lib, bstride=100) == B.PKV_ERR_INVALID_ARG
    assert _write(lib, T=-1) == B.PKV_ERR_INVALID_ARG
    assert _write(lib, nb=0) == B.PKV_ERR_INVALID_ARG
    # an empty batch is a successful no-op, even with NULL inputs
    assert _write(lib, T=0, key=NULL, value=NULL, slots=NULL) == B.PKV_OK
    assert B.last_error() == ""


def _slots_unique(lib, **kw):
    a = dict(slots=FAKE, T=4, nb=8, bs=16, marks=FAKE, mbytes=16)
    a.update(kw)
    return lib.pkv_check_slots_unique(a["slots"], a["T"], a["nb"], a["bs"], a["marks"],
                                      a["mbytes"], NULL)


def test_slots_unique_rejections(lib):
    """Argument checks of the duplicate-slot check (8 blocks of 16 slots -> 4 words, 16 bytes)."""
    assert _slots_unique(lib, slots=NULL) == B.PKV_ERR_INVALID_ARG
    assert "NULL" in B.last_error()
    assert _slots_unique(lib, marks=NULL) == B.PKV_ERR_INVALID_ARG
    assert _slots_unique(lib, mbytes=15) == B.PKV_ERR_INVALID_ARG
    assert "16 bytes" in B.last_error()
    assert _slots_unique(lib, nb=9) == B.PKV_ERR_INVALID_ARG       # 144 slots need 20 bytes
    assert _slots_unique(lib, marks=ctypes.c_void_p(FAKE.value + 2)) == B.PKV_ERR_INVALID_ARG
    assert "aligned" in B.last_error()
    assert _slots_unique(lib, bs=12) == B.PKV_ERR_INVALID_ARG
    assert _slots_unique(lib, nb=0) == B.PKV_ERR_INVALID_ARG
    assert _slots_unique(lib, T=-1) == B.PKV_ERR_INVALID_ARG
    assert _slots_unique(lib, T=0, slots=NULL, marks=NULL) == B.PKV_OK
    assert B.last_error() == ""


def _decode(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bstride=16 * 8 * 128, bt=FAKE, mb=256, sl=FAKE,
             S=64, H=32, Hkv=8, D=128, nb=9000, bs=16, scale=0.088, maxL=4096, ws=FAKE, wsb=0,
             dt=B.PKV_BF16)
    a.update(kw)
    return lib.pkv_paged_attention_decode(a["out"], a["q"], a["kc"], a["vc"], a["bstride"], a["bt"],
                                          a["mb"], a["sl"], a["S"], a["H"], a["Hkv"], a["D"],
                                          a["nb"], a["bs"], a["scale"], a["maxL"], a["ws"],
                                          a["wsb"], a["dt"], NULL)


def test_decode_rejections(lib):
    need = lib.pkv_decode_workspace_size(64, 32, 8, 128, 16, 4096)
    assert need > 0
    assert _decode(lib, wsb=need - 1) == B.PKV_ERR_WORKSPACE
    assert _decode(lib, ws=NULL, wsb=need) == B.PKV_ERR_WORKSPACE
    assert "workspace" in B.last_error()
    assert _decode(lib, H=30) == B.PKV_ERR_INVALID_ARG
    assert "multiple" in B.last_error()
    assert _decode(lib, out=NULL, wsb=need) == B.PKV_ERR_INVALID_ARG
    assert _decode(lib, D=80, bstride=16 * 8 * 80) == B.PKV_ERR_UNSUPPORTED
    assert _decode(lib, mb=100, wsb=need) == B.PKV_ERR_INVALID_ARG      # 100*16 < 4096
    assert _decode(lib, scale=float("nan"), wsb=need) == B.PKV_ERR_INVALID_ARG
    assert _decode(lib, S=0) == B.PKV_OK


def test_decode_rejects_misaligned_workspace(lib):
    """The partials are stored as 16-byte vectors and the planning tables as int64: a
    workspace that is not 16-byte aligned is rejected on the host."""
    need = lib.pkv_decode_workspace_size(64, 32, 8, 128, 16, 4096)
    assert _decode(lib, ws=ctypes.c_void_p(0x1008), wsb=need) == B.PKV_ERR_INVALID_ARG
    assert "aligned" in B.last_error()
    # a plan without a workspace ignores the pointer
    assert lib.pkv_decode_workspace_size(64, 32, 8, 128, 16, 256) == 0


def _noalloc(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bstride=16 * 8 * 128, bt=FAKE, mb=256, sl=FAKE,
             S=64, H=32, Hkv=8, D=128, nb=9000, bs=16, scale=0.088, maxL=4096, dt=B.PKV_BF16)
    a.update(kw)
    return lib.pkv_paged_attention_decode_noalloc(a["out"], a["q"], a["kc"], a["vc"], a["bstride"],
                                                  a["bt"], a["mb"], a["sl"], a["S"], a["H"],
                                                  a["Hkv"], a["D"], a["nb"], a["bs"], a["scale"],
                                                  a["maxL"], a["dt"], NULL)


def test_decode_noalloc_rejections(lib):
    """The allocation-free decode rejects, before it looks up its scratch array, sizes
    whose workspace exceeds that array, and every argument the plain decode rejects."""
    limit = 16 << 20
    # 2M sequences: 8.5 MB of partials plus 16 MB of planning tables
    need = lib.pkv_decode_workspace_size(2_000_000, 64, 8, 128, 16, 5000)
    assert need > limit
    assert _noalloc(lib, S=2_000_000, H=64, maxL=5000, mb=400) == B.PKV_ERR_WORKSPACE
    assert "scratch" in B.last_error()
    # the decode batch fits
    assert lib.pkv_decode_workspace_size(64, 32, 8, 128, 16, 4096) <= limit
    assert _noalloc(lib, dt=7) == B.PKV_ERR_UNSUPPORTED
    assert _noalloc(lib, S=0) == B.PKV_OK


def test_mixed_rejects_misaligned_workspace(lib):
    need = lib.pkv_mixed_workspace_size(64, 32, 8, 128, 16, 4096)
    assert need > 0
    rc = lib.pkv_paged_attention_mixed(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16 * 8 * 128, FAKE, 256,
                                       66, 64 + 100, 2, 100, 32, 8, 128, 9000, 16, 0.088,
                                       B.PKV_MASK_CAUSAL, 0, 50, 4096, ctypes.c_void_p(0x1004),
                                       need, B.PKV_BF16, NULL)
    assert rc == B.PKV_ERR_INVALID_ARG
    assert "aligned" in B.last_error()


def test_decode_rejects_workspace_without_prefix_tables(lib):
    """Beyond 256 sequences a workspace sized for the partials alone is too small: the
    call fails on the host, before any launch."""
    part = 32 * 128 * 2 * 130 * 4           # the partials (what 256 sequences need)
    need = lib.pkv_decode_workspace_size(2000, 32, 8, 128, 16, 4096)
    assert need == part + (2000 + 1 + 128) * 8 + 128 * 4
    assert _decode(lib, S=2000, wsb=part) == B.PKV_ERR_WORKSPACE
    assert "workspace" in B.last_error()


def test_decode_workspace_prefix_tables(lib):
    """Stream mode beyond 256 sequences adds the planning tables (int64 prefix sums per
    sequence plus one, int64 start and int32 first sequence per range); 256 sequences
    scan without them.  The generation rows of a mixed batch take the decode plan."""
    part = 8 * 128 * 2 * 130 * 4            # 8 heads x 128 ranges x 2 slots x (D + 2) floats
    assert lib.pkv_decode_workspace_size(256, 8, 8, 128, 16, 5000) == part
    assert lib.pkv_decode_workspace_size(257, 8, 8, 128, 16, 5000) == \
        part + (257 + 1 + 128) * 8 + 128 * 4
    assert lib.pkv_decode_workspace_size(1025, 8, 8, 128, 16, 5000) == \
        part + (1025 + 1 + 128) * 8 + 128 * 4
    # mixed batch: the decode workspace of its generation rows
    for n in (100, 1000, 1500):
        assert lib.pkv_mixed_workspace_size(n, 8, 8, 128, 16, 5000) == \
            lib.pkv_decode_workspace_size(n, 8, 8, 128, 16, 5000)
    # all sequences within one split: no partials, no tables, whatever the batch size
    assert lib.pkv_decode_workspace_size(5000, 8, 8, 128, 16, 256) == 0


def test_decode_workspace_size_plan(lib):
    # one split per sequence -> no workspace
    assert lib.pkv_decode_workspace_size(30720, 16, 16, 128, 16, 16) == 0
    # stream mode: 1024 waves over 8 wave groups (4 heads a wave) = 128 key ranges;
    # 32 heads x 128 ranges x 2 partial slots x (128 + 2) floats
    assert lib.pkv_decode_workspace_size(64, 32, 8, 128, 16, 4096) == 32 * 128 * 2 * 130 * 4
    # beyond 256 sequences stream mode adds the planning tables: 128 ranges (1024 waves,
    # 8 wave groups), partials 8 heads x 128 x 2 slots, then int64 cu[S + 1], int64
    # rpos[128], int32 rstart[128]
    assert lib.pkv_decode_workspace_size(2000, 8, 8, 128, 16, 5000) == \
        8 * 128 * 2 * 130 * 4 + (2000 + 1 + 128) * 8 + 128 * 4
    assert lib.pkv_decode_workspace_size(2000, 8, 8, 128, 16, 300) == 0
    assert lib.pkv_decode_workspace_size(64, 30, 8, 128, 16, 4096) == 0    # invalid -> 0
    assert lib.pkv_decode_workspace_size(1, 8, 8, 128, 16, 131072) > 0


def _prefill(lib, **kw):
    a = dict(out=FAKE, q=FAKE, cu=FAKE, sl=FAKE, kc=FAKE, vc=FAKE, bstride=16 * 8 * 128, bt=FAKE,
             mb=512, S=4, T=32768, H=64, Hkv=8, D=128, nb=2049, bs=16, scale=0.088,
             mask=B.PKV_MASK_BLOCK_CAUSAL, span=2048, maxq=8192, maxL=8192, dt=B.PKV_BF16)
    a.update(kw)
    return lib.pkv_paged_attention_prefill(a["out"], a["q"], a["cu"], a["sl"], a["kc"], a["vc"],
                                           a["bstride"], a["bt"], a["mb"], a["S"], a["T"], a["H"],
                                           a["Hkv"], a["D"], a["nb"], a["bs"], a["scale"],
                                           a["mask"], a["span"], a["maxq"], a["maxL"], a["dt"],
                                           NULL)


def test_prefill_rejections(lib):
    assert _prefill(lib, span=0) == B.PKV_ERR_INVALID_ARG
    assert "span_len" in B.last_error()
    assert _prefill(lib, mask=5) == B.PKV_ERR_INVALID_ARG
    assert _prefill(lib, H=60) == B.PKV_ERR_INVALID_ARG
    assert _prefill(lib, cu=NULL) == B.PKV_ERR_INVALID_ARG
    assert _prefill(lib, maxq=9000) == B.PKV_ERR_INVALID_ARG            # > max_seq_len
    assert _prefill(lib, T=40000) == B.PKV_ERR_INVALID_ARG              # > S * max_q_len
    assert _prefill(lib, mb=100) == B.PKV_ERR_INVALID_ARG
    assert _prefill(lib, D=32, bstride=16 * 8 * 32) == B.PKV_ERR_UNSUPPORTED
    assert _prefill(lib, dt=3) == B.PKV_ERR_UNSUPPORTED
    assert _prefill(lib, T=0) == B.PKV_OK


def test_gather_rejections(lib):
    r = lib.pkv_kv_cache_gather(NULL, FAKE, FAKE, FAKE, FAKE, 16 * 256, FAKE, 4, 2, 10, 8, 16, 2,
                                128, 40, B.PKV_BF16, NULL)
    assert r == B.PKV_ERR_INVALID_ARG
    r = lib.pkv_kv_cache_gather(FAKE, FAKE, FAKE, FAKE, FAKE, 16 * 256, FAKE, 2, 2, 10, 8, 16, 2,
                                128, 40, B.PKV_BF16, NULL)
    assert r == B.PKV_ERR_INVALID_ARG                                   # 2*16 < 40


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError):
        B.load(str(tmp_path / "missing.so"))


def test_device_checks_switch(lib):
    """The switch needs no GPU; reading the error word does (covered by the GPU tests)."""
    assert lib.pkv_set_device_checks(1) == B.PKV_OK
    assert lib.pkv_set_device_checks(0) == B.PKV_OK
    assert B.last_error() == ""


def _write_fp8(lib, **kw):
    a = dict(key=FAKE, value=FAKE, stride=1024, slots=FAKE, T=10, kc=FAKE, vc=FAKE,
             bstride=16 * 1024, nb=4, bs=16, hkv=8, d=128, ks=0.02, vs=0.03, dt=B.PKV_BF16)
    a.update(kw)
    return lib.pkv_kv_cache_write_fp8(a["key"], a["value"], a["stride"], a["slots"], a["T"],
                                      a["kc"], a["vc"], a["bstride"], a["nb"], a["bs"], a["hkv"],
                                      a["d"], a["ks"], a["vs"], a["dt"], NULL)


def test_write_fp8_rejections(lib):
    assert _write_fp8(lib, ks=0.0) == B.PKV_ERR_INVALID_ARG
    assert "scale" in B.last_error()
    assert _write_fp8(lib, vs=-1.0) == B.PKV_ERR_INVALID_ARG
    assert _write_fp8(lib, ks=float("inf")) == B.PKV_ERR_INVALID_ARG
    assert _write_fp8(lib, ks=float("nan")) == B.PKV_ERR_INVALID_ARG
    assert _write_fp8(lib, ks=1e-45) == B.PKV_ERR_INVALID_ARG           # 1/scale overflows
    assert _write_fp8(lib, dt=B.PKV_FP8_E4M3) == B.PKV_ERR_UNSUPPORTED  # source must be a float
    assert _write_fp8(lib, stride=1026) == B.PKV_ERR_INVALID_ARG        # not a multiple of 4
    assert _write_fp8(lib, key=ctypes.c_void_p(0x1002)) == B.PKV_ERR_INVALID_ARG
    assert "aligned" in B.last_error()
    assert _write_fp8(lib, kc=ctypes.c_void_p(0x1001)) == B.PKV_ERR_INVALID_ARG
    assert _write_fp8(lib, key=NULL) == B.PKV_ERR_INVALID_ARG
    assert _write_fp8(lib, T=0, key=NULL, value=NULL, slots=NULL) == B.PKV_OK


def _decode_fp8(lib, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bstride=16 * 8 * 128, bt=FAKE, mb=256, sl=FAKE,
             S=64, H=32, Hkv=8, D=128, nb=9000, bs=16, scale=0.088, ks=0.02, vs=0.03, maxL=4096,
             ws=FAKE, wsb=1 << 30, dt=B.PKV_BF16)
    a.update(kw)
    return lib.pkv_paged_attention_decode_fp8(a["out"], a["q"], a["kc"], a["vc"], a["bstride"],
                                              a["bt"], a["mb"], a["sl"], a["S"], a["H"], a["Hkv"],
                                              a["D"], a["nb"], a["bs"], a["scale"], a["ks"],
                                              a["vs"], a["maxL"], a["ws"], a["wsb"], a["dt"], NULL)


def test_decode_fp8_rejections(lib):
    assert _decode_fp8(lib, dt=B.PKV_F32) == B.PKV_ERR_UNSUPPORTED
    assert _decode_fp8(lib, dt=B.PKV_FP8_E4M3) == B.PKV_ERR_UNSUPPORTED
    assert _decode_fp8(lib, ks=0.0) == B.PKV_ERR_INVALID_ARG
    assert _decode_fp8(lib, vs=float("inf")) == B.PKV_ERR_INVALID_ARG
    assert _decode_fp8(lib, bstride=16 * 8 * 128 + 8) == B.PKV_ERR_INVALID_ARG   # 16-byte rows
    assert "16" in B.last_error()
    assert _decode_fp8(lib, kc=ctypes.c_void_p(0x1008)) == B.PKV_ERR_INVALID_ARG
    assert _decode_fp8(lib, wsb=0) == B.PKV_ERR_WORKSPACE
    assert _decode_fp8(lib, H=30) == B.PKV_ERR_INVALID_ARG
    assert _decode_fp8(lib, S=0) == B.PKV_OK


def test_attention_alignment_rejections(lib):
    """The attention calls read rows in 16-byte vectors: misaligned pointers or block
    strides are rejected on the host."""
    need = lib.pkv_decode_workspace_size(64, 32, 8, 128, 16, 4096)
    assert _decode(lib, q=ctypes.c_void_p(0x1002), wsb=need) == B.PKV_ERR_INVALID_ARG
    assert _decode(lib, bstride=16 * 8 * 128 + 4, wsb=need) == B.PKV_ERR_INVALID_ARG
    assert _decode(lib, bstride=16 * 8 * 128 + 2, dt=B.PKV_F32, wsb=need) == B.PKV_ERR_INVALID_ARG
    assert _prefill(lib, out=ctypes.c_void_p(0x1004)) == B.PKV_ERR_INVALID_ARG
    assert _prefill(lib, bstride=16 * 8 * 128 + 2) == B.PKV_ERR_INVALID_ARG


def test_gather_takes_fp8_codes(lib):
    """The gather is a byte copy for FP8 caches: PKV_FP8_E4M3 passes the dtype check (and
    then fails on the NULL output here)."""
    r = lib.pkv_kv_cache_gather(NULL, FAKE, FAKE, FAKE, FAKE, 16 * 256, FAKE, 4, 2, 10, 8, 16,
                                2, 128, 40, B.PKV_FP8_E4M3, NULL)
    assert r == B.PKV_ERR_INVALID_ARG and "NULL" in B.last_error()
    r = lib.pkv_kv_cache_gather(NULL, FAKE, FAKE, FAKE, FAKE, 16 * 256, FAKE, 4, 2, 10, 8, 16,
                                2, 128, 40, 9, NULL)
    assert r == B.PKV_ERR_UNSUPPORTED


def _prefill_fp8(lib, **kw):
    a = dict(out=FAKE, q=FAKE, cu=FAKE, sl=FAKE, kc=FAKE, vc=FAKE, bstride=16 * 8 * 128, bt=FAKE,
             mb=512, S=4, T=32768, H=64, Hkv=8, D=128, nb=2049, bs=16, scale=0.088, ks=0.02,
             vs=0.03, mask=B.PKV_MASK_BLOCK_CAUSAL, span=2048, maxq=8192, maxL=8192,
             dt=B.PKV_BF16)
    a.update(kw)
    return lib.pkv_paged_attention_prefill_fp8(a["out"], a["q"], a["cu"], a["sl"], a["kc"],
                                               a["vc"], a["bstride"], a["bt"], a["mb"], a["S"],
                                               a["T"], a["H"], a["Hkv"], a["D"], a["nb"], a["bs"],
                                               a["scale"], a["ks"], a["vs"], a["mask"], a["span"],
                                               a["maxq"], a["maxL"], a["dt"], NULL)


def test_prefill_fp8_rejections(lib):
    assert _prefill_fp8(lib, dt=B.PKV_F32) == B.PKV_ERR_UNSUPPORTED
    assert _prefill_fp8(lib, ks=-0.5) == B.PKV_ERR_INVALID_ARG
    assert _prefill_fp8(lib, vs=0.0) == B.PKV_ERR_INVALID_ARG
    assert _prefill_fp8(lib, mask=3) == B.PKV_ERR_INVALID_ARG          # no span lists on FP8
    assert _prefill_fp8(lib, span=0) == B.PKV_ERR_INVALID_ARG
    assert _prefill_fp8(lib, bstride=16 * 8 * 128 + 8) == B.PKV_ERR_INVALID_ARG
    assert _prefill_fp8(lib, cu=NULL) == B.PKV_ERR_INVALID_ARG
    assert _prefill_fp8(lib, T=0) == B.PKV_OK


def test_smallseq_rejections(lib):
    def fwd(**kw):
        a = dict(out=FAKE, w=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bstride=16 * 16 * 128, bt=FAKE, mb=1,
                 sl=FAKE, S=30720, H=16, Hkv=16, D=128, nb=30721, bs=16, scale=0.088, maxL=16,
                 dt=B.PKV_BF16)
        a.update(kw)
        return lib.pkv_smallseq_attention_fwd(a["out"], a["w"], a["q"], a["kc"], a["vc"],
                                              a["bstride"], a["bt"], a["mb"], a["sl"], a["S"],
                                              a["H"], a["Hkv"], a["D"], a["nb"], a["bs"],
                                              a["scale"], a["maxL"], a["dt"], NULL)
    assert fwd(maxL=17) == B.PKV_ERR_INVALID_ARG
    assert "16" in B.last_error()
    assert fwd(maxL=0) == B.PKV_ERR_INVALID_ARG
    assert fwd(dt=B.PKV_F32) == B.PKV_ERR_UNSUPPORTED
    assert fwd(D=80, bstride=16 * 16 * 80) == B.PKV_ERR_UNSUPPORTED
    assert fwd(w=NULL) == B.PKV_ERR_INVALID_ARG
    assert fwd(H=12, Hkv=8) == B.PKV_ERR_INVALID_ARG
    assert fwd(S=0) == B.PKV_OK
    r = lib.pkv_smallseq_attention_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       16 * 16 * 128, FAKE, 1, FAKE, NULL, 4, 40, 16, 16, 128,
                                       5, 16, 0.088, 16, B.PKV_BF16, NULL)
    assert r == B.PKV_ERR_INVALID_ARG and "cu_seq_lens" in B.last_error()


def test_launch_log_switch(lib):
    """The launch-log switch needs no GPU (the lines themselves are checked on the GPU)."""
    assert lib.pkv_set_log(1) == B.PKV_OK
    assert lib.pkv_set_log(0) == B.PKV_OK
