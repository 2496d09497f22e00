"""The C-ABI library loads, exports every symbol include/osdn.h declares, and
rejects malformed arguments on the host (no GPU work is started here)."""
import ctypes
import os
import re

import pytest

import preconditioned_delta_rule_amd as osdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "osdn.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(osdn_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(osdn.library_path()):
        pytest.fail("libosdn.so is not built; run __graft_entry__.build() first")
    return osdn.load()


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert len(syms) >= 9
    for s in syms:
        assert hasattr(lib, s), "libosdn.so does not export %s" % s
    assert set(syms) == set(osdn.SYMBOLS)


def test_desc_layout_and_defaults(lib):
    d = osdn.Desc()
    assert lib.osdn_desc_init(ctypes.byref(d), 4, 4096, 16, 128, 128) == osdn.OK
    assert (d.B, d.T, d.H, d.K, d.V) == (4, 4096, 16, 128, 128)
    assert d.chunk == 64 and d.dtype == osdn.BF16 and d.clamp == 1 and d.beta_aware == 1
    assert d.eta == pytest.approx(0.003) and d.eps == pytest.approx(1e-6)
    assert (d.d_min, d.d_max, d.q_scale) == (0.5, 2.0, 1.0)
    assert ctypes.sizeof(osdn.Desc) == 88 and d.r_per_key == 0 and d.o_f32 == 0
    assert lib.osdn_validate(ctypes.byref(d)) == osdn.OK
    assert lib.osdn_version() >> 16 == 1


def test_status_strings(lib):
    names = [lib.osdn_status_str(i).decode() for i in range(4)]
    assert names == ["OSDN_OK", "OSDN_EINVAL", "OSDN_EUNSUPPORTED", "OSDN_EHIP"]


BAD = [
    (dict(B=0), osdn.EINVAL), (dict(H=0), osdn.EINVAL), (dict(T=-1), osdn.EINVAL),
    (dict(K=0), osdn.EINVAL), (dict(V=0), osdn.EINVAL), (dict(chunk=0), osdn.EINVAL),
    (dict(chunk=65), osdn.EUNSUPPORTED), (dict(K=129), osdn.EUNSUPPORTED),
    (dict(V=200), osdn.EUNSUPPORTED), (dict(H=65537), osdn.EUNSUPPORTED), (dict(dtype=7), osdn.EINVAL),
    (dict(eta=-1.0), osdn.EINVAL), (dict(eps=0.0), osdn.EINVAL),
    (dict(d_min=2.0, d_max=1.0), osdn.EINVAL), (dict(d_min=0.0), osdn.EINVAL),
    (dict(q_scale=float("inf")), osdn.EINVAL), (dict(eta=float("nan")), osdn.EINVAL),
    (dict(r_per_key=2), osdn.EINVAL), (dict(o_f32=2), osdn.EINVAL),
]


@pytest.mark.parametrize("change,status", BAD)
def test_validation_rejects(lib, change, status):
    d = osdn.Desc()
    lib.osdn_desc_init(ctypes.byref(d), 2, 16, 2, 16, 16)
    for k, v in change.items():
        setattr(d, k, v)
    assert lib.osdn_validate(ctypes.byref(d)) == status
    assert lib.osdn_last_error().decode() != ""
    assert lib.osdn_fwd_workspace_bytes(ctypes.byref(d)) == 0


def test_box_unchecked_without_clamp(lib):
    d = osdn.Desc()
    lib.osdn_desc_init(ctypes.byref(d), 1, 8, 1, 16, 16)
    d.clamp, d.d_min, d.d_max = 0, 3.0, 1.0
    assert lib.osdn_validate(ctypes.byref(d)) == osdn.OK


def test_scan_only_limits(lib):
    # phase 1 alone accepts K up to 256, phase 2 does not
    d = osdn.Desc()
    lib.osdn_desc_init(ctypes.byref(d), 1, 8, 1, 256, 16)
    assert lib.osdn_validate(ctypes.byref(d)) == osdn.EUNSUPPORTED
    d.K = 300
    null = ctypes.c_void_p(None)
    st = lib.osdn_precond_scan(ctypes.byref(d), null, null, null, null, null, null, null,
                               ctypes.c_size_t(0), null)
    assert st == osdn.EUNSUPPORTED
    assert lib.osdn_precond_scan_workspace_bytes(ctypes.byref(d)) == 0
    assert lib.osdn_precond_scan_counters_offset(ctypes.byref(d)) == -1


def test_head_limit_is_phase2_only(lib):
    # the sweep's 32-bit row offsets bound H for phase 2; phase 1 alone has no such bound
    null = ctypes.c_void_p(None)
    d = osdn.Desc()
    lib.osdn_desc_init(ctypes.byref(d), 1, 0, 65536, 16, 16)
    assert lib.osdn_validate(ctypes.byref(d)) == osdn.OK
    d.H = 65537
    st = lib.osdn_chunk_fwd(ctypes.byref(d), null, null, null, null, null, null, null, null, null,
                            null, ctypes.c_size_t(0), null)
    assert st == osdn.EUNSUPPORTED
    assert lib.osdn_precond_scan_workspace_bytes(ctypes.byref(d)) > 0


def test_null_and_misaligned_pointers_rejected_before_launch(lib):
    d = osdn.Desc()
    lib.osdn_desc_init(ctypes.byref(d), 1, 8, 1, 16, 16)
    null = ctypes.c_void_p(None)
    z = ctypes.c_size_t(0)
    st = lib.osdn_precond_scan(ctypes.byref(d), null, null, null, null, null, null, null, z, null)
    assert st == osdn.EINVAL and "k must not be NULL" in lib.osdn_last_error().decode()
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1004)
    st = lib.osdn_precond_scan(ctypes.byref(d), fake, odd, null, null, fake, null, null, z, null)
    assert st == osdn.EINVAL and "aligned" in lib.osdn_last_error().decode()
    st = lib.osdn_precond_scan(ctypes.byref(d), fake, fake, null, null, ctypes.c_void_p(0x2000),
                               null, odd, ctypes.c_size_t(1 << 20), null)
    assert st == osdn.EINVAL and "workspace is not" in lib.osdn_last_error().decode()
    st = lib.osdn_precond_scan(ctypes.byref(d), fake, fake, null, null, ctypes.c_void_p(0x2000),
                               null, ctypes.c_void_p(0x3000), ctypes.c_size_t(16), null)
    assert st == osdn.EINVAL and "needed" in lib.osdn_last_error().decode()
    st = lib.osdn_chunk_fwd(ctypes.byref(d), fake, fake, fake, fake, fake, null, null, fake,
                            null, null, z, null)
    assert st == osdn.EINVAL and "alias" in lib.osdn_last_error().decode()
    st = lib.osdn_fwd(ctypes.byref(d), fake, fake, fake, fake, null, null, null, null,
                      ctypes.c_void_p(0x2000), null, null, null, null, ctypes.c_size_t(0), null)
    assert st == osdn.EINVAL and "workspace" in lib.osdn_last_error().decode()
    st = lib.osdn_fwd(ctypes.byref(d), fake, fake, fake, fake, null, null, null, null,
                      ctypes.c_void_p(0x2000), null, null, null, ctypes.c_void_p(0x3000),
                      ctypes.c_size_t(16), null)
    assert st == osdn.EINVAL and "needed" in lib.osdn_last_error().decode()


def test_workspace_bytes(lib):
    # chunked phase 1 at B=4, T=4096, H=16, K=128: key norms and step scalars
    # (fp32 per token), d at each of the 64 chunk starts, a word and a 64-bit
    # token mask per chunk, three counters per (b,h), then a flag word and a
    # 64 x 64 fp32 triangular factor per chunk, each region rounded up to 256
    # bytes
    d = osdn.Desc()
    lib.osdn_desc_init(ctypes.byref(d), 4, 4096, 16, 128, 128)
    tok = 4 * 4096 * 16 * 4
    counters = 2 * tok + 4 * 16 * 64 * 128 * 4 + 4 * 16 * 64 * 4 + 4 * 16 * 64 * 8
    scan = counters + 256 * 3 + 4 * 16 * 64 * 4 + 4 * 16 * 64 * 64 * 64 * 4
    assert lib.osdn_precond_scan_workspace_bytes(ctypes.byref(d)) == scan
    assert lib.osdn_precond_scan_counters_offset(ctypes.byref(d)) == counters
    # phase 2 on the matrix cores keeps, per chunk, the six 16 x 32 blocks of
    # (I + A)^-1 on and below the diagonal (bf16: each lane's 4 + 4 columns of
    # two 16-wide halves), the intra-chunk scores in the same blocks as hi/lo
    # bf16 pairs, and beta and the two decay factors e^g_t, e^(g_L - g_t) (fp32)
    wy = 4 * 16 * 64 * (6 * 16 * 32 * 2 * 3 + 3 * 64 * 4)
    assert lib.osdn_chunk_fwd_workspace_bytes(ctypes.byref(d)) == wy
    assert lib.osdn_fwd_workspace_bytes(ctypes.byref(d)) == 4 * 4096 * 16 * 128 * 2 + scan + wy
    d.dtype = osdn.F32
    assert lib.osdn_chunk_fwd_workspace_bytes(ctypes.byref(d)) == 0
    assert lib.osdn_fwd_workspace_bytes(ctypes.byref(d)) == 4 * 4096 * 16 * 128 * 4 + scan
    # a ragged tail chunk counts as a chunk
    d.T = 4097
    n = 65
    tok = -(-4 * 4097 * 16 * 4 // 256) * 256
    scan = (2 * tok + 4 * 16 * n * 128 * 4 + -(-4 * 16 * n * 4 // 256) * 256
            + -(-4 * 16 * n * 8 // 256) * 256 + 256 * 3
            + -(-4 * 16 * n * 4 // 256) * 256 + 4 * 16 * n * 64 * 64 * 4)
    assert lib.osdn_precond_scan_workspace_bytes(ctypes.byref(d)) == scan


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(osdn, "_lib", None)
    monkeypatch.setattr(osdn, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="libosdn.so not found"):
        osdn.load()


def test_profile_end_without_begin_is_rejected(lib):
    n = ctypes.c_int(-1)
    st = lib.osdn_profile_end(None, None, 0, ctypes.byref(n))
    assert st == osdn.EINVAL and "no profile" in lib.osdn_last_error().decode()


def test_decode_argument_checks(lib):
    # decode: at most OSDN_DECODE_MAX_T tokens, required pointers, no aliasing
    # of outputs with other inputs; all rejected on the host before any launch
    null = ctypes.c_void_p(None)
    fake, fake2, fake3 = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    d = osdn.Desc()
    lib.osdn_desc_init(ctypes.byref(d), 2, osdn.DECODE_MAX_T + 1, 4, 128, 128)
    args = [fake, fake, fake, fake2, null, null, null, null, fake3, null, null, null]
    assert lib.osdn_decode(ctypes.byref(d), *args) == osdn.EUNSUPPORTED
    assert "at most" in lib.osdn_last_error().decode()
    d.T = 1
    st = lib.osdn_decode(ctypes.byref(d), fake, null, fake, fake2, null, null, null, null, fake3,
                         null, null, null)
    assert st == osdn.EINVAL and "k must not be NULL" in lib.osdn_last_error().decode()
    st = lib.osdn_decode(ctypes.byref(d), fake, fake, fake, fake2, null, null, null, null, fake,
                         null, null, null)
    assert st == osdn.EINVAL and "alias" in lib.osdn_last_error().decode()
    st = lib.osdn_decode(ctypes.byref(d), fake, fake, fake, fake2, null, null, ctypes.c_void_p(0x4000),
                         null, fake3, ctypes.c_void_p(0x4000), null, null)
    assert st == osdn.EINVAL and "S_out may alias S0 only" in lib.osdn_last_error().decode()
    st = lib.osdn_decode(ctypes.byref(d), fake, fake, fake, fake2, null, null, null, null, fake3,
                         null, ctypes.c_void_p(0x4004), null)
    assert st == osdn.EINVAL and "aligned" in lib.osdn_last_error().decode()
    d.K = 129
    assert lib.osdn_decode(ctypes.byref(d), *args) == osdn.EUNSUPPORTED


def test_size_queries_return_64_bit(lib):
    # workspace sizes above 2^31 bytes come back whole through the binding
    assert osdn.bwd_workspace_bytes(4, 4096, 16, 128, 128) > 2 ** 31
    assert osdn.fwd_workspace_bytes(256, 4096, 16, 128, 128) > 2 ** 32


def test_kda_argument_checks(lib):
    # OSKDA: sizes, required pointers, aliasing and workspace, all on the host
    null = ctypes.c_void_p(None)
    fake, fake2, fake3 = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    d = osdn.Desc()
    lib.osdn_desc_init(ctypes.byref(d), 2, 100, 4, 128, 128)
    z = ctypes.c_size_t(0)
    st = lib.osdn_kda_fwd(ctypes.byref(d), fake, fake, fake, fake2, null, null, null, null, fake3,
                          null, null, null, null, z, null)
    assert st == osdn.EINVAL and "workspace" in lib.osdn_last_error().decode()
    st = lib.osdn_kda_fwd(ctypes.byref(d), fake, fake, fake, fake2, null, null, null, null, fake,
                          null, null, null, fake3, z, null)
    assert st == osdn.EINVAL and "alias" in lib.osdn_last_error().decode()
    st = lib.osdn_kda_fwd(ctypes.byref(d), fake, null, fake, fake2, null, null, null, null, fake3,
                          null, null, null, fake3, z, null)
    assert st == osdn.EINVAL and "k must not be NULL" in lib.osdn_last_error().decode()
    need = lib.osdn_kda_fwd_workspace_bytes(ctypes.byref(d))
    # 2 x 4 heads x 2 chunks of 64 tokens: 128.5 KiB of operands each, plus phase 1's share
    assert need >= 16 * (3 * 64 * 128 + 2 * 64 * 64 + 128) * 4
    st = lib.osdn_kda_fwd(ctypes.byref(d), fake, fake, fake, fake2, null, null, null, null, fake3,
                          null, null, null, ctypes.c_void_p(0x10000), ctypes.c_size_t(need - 1), null)
    assert st == osdn.EINVAL and "needed" in lib.osdn_last_error().decode()
    d.V = 129
    assert lib.osdn_kda_fwd_workspace_bytes(ctypes.byref(d)) == 0
    st = lib.osdn_kda_fwd(ctypes.byref(d), fake, fake, fake, fake2, null, null, null, null, fake3,
                          null, null, null, fake3, z, null)
    assert st == osdn.EUNSUPPORTED


def test_vector_retention_rejected_where_unsupported(lib):
    null = ctypes.c_void_p(None)
    fake, fake2, fake3 = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    d = osdn.Desc()
    lib.osdn_desc_init(ctypes.byref(d), 1, 4, 2, 16, 16)
    d.r_per_key = 1
    st = lib.osdn_decode(ctypes.byref(d), fake, fake, fake, fake2, fake2, null, null, null, fake3,
                         null, null, null)
    assert st == osdn.EUNSUPPORTED and "retention" in lib.osdn_last_error().decode()
    args = [fake, fake, fake, fake2, fake2] + [null] * 15 + [ctypes.c_size_t(0), null]
    assert lib.osdn_bwd(ctypes.byref(d), *args) == osdn.EUNSUPPORTED
