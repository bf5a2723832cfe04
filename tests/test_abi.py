"""The C-ABI library loads, exports every declared symbol, and rejects invalid
arguments on the host before touching the GPU.  Runs on the CPU: no call
here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import head_latent_attention_cache_amd as mla
from head_latent_attention_cache_amd import _lib
from mla_inputs import CONFIGS, SMALL_CONFIGS, get_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")
PROBE_HEADER = os.path.join(ROOT, "include", "mla_probe.h")


def _declared(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"mla_cache_append", "mla_absorb_q", "mla_attention", "mla_unabsorb_out"} <= names
    assert names == set(_lib.SIGNATURES), names ^ set(_lib.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n
    assert not any(n.startswith("mla_probe") for n in names)


def test_probe_library_exports_its_header():
    """The measurement probes live in their own library, off the MLA ABI."""
    plib = _lib.load_probe()
    names = _declared(PROBE_HEADER)
    assert names == set(_lib.PROBE_SIGNATURES), names ^ set(_lib.PROBE_SIGNATURES)
    for n in names:
        assert hasattr(plib, n), n
    mla_lib = _lib.load()
    assert not hasattr(mla_lib, "mla_probe_mfma") and not hasattr(mla_lib, "mla_probe_hbm_read")


def test_version_and_status_strings(lib):
    assert lib.mla_abi_version() == 1
    assert lib.mla_status_string(0) == b"MLA_OK"
    assert lib.mla_status_string(-1) == b"MLA_ERR_INVALID_ARG"
    assert lib.mla_status_string(-3) == b"MLA_ERR_WORKSPACE"


def _dims(cfg, **kw):
    d = mla.api.dims_from_config(cfg)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _geom(cfg, **kw):
    g = mla.api.geom_from_config(cfg)
    for k, v in kw.items():
        setattr(g, k, v)
    return g


@pytest.mark.parametrize("key", [1, 2, 3, 4, 5, 6])
def test_cache_sizes(lib, key):
    cfg = get_config(key)
    d, g = _dims(cfg), _geom(cfg)
    nb = lib.mla_cache_bytes(ctypes.byref(d), ctypes.byref(g))
    na = lib.mla_cache_aux_bytes(ctypes.byref(d), ctypes.byref(g))
    rows = cfg.batch * cfg.capacity
    if cfg.cache_fmt == "int4":
        assert nb == rows * cfg.d_qk // 2
        assert na == rows * (cfg.d_c // 32 + 1) * 2
        assert (nb + na) // rows == 322
    elif cfg.cache_fmt == "int2":
        # 2-bit content codes, 4-bit rotary codes, fp16 group and token scales
        assert nb == rows * (cfg.d_c // 4 + cfg.d_r // 2)
        assert na == rows * (cfg.d_c // 32 + 1) * 2
        assert (nb + na) // rows == 194
    else:
        assert nb == rows * cfg.d_qk * (2 if cfg.dtype == "bf16" else 4)
        assert na == 0


BAD_DIMS = [
    ("d_r odd", dict(d_r=15)),
    ("bands do not sum to d_r", dict(band=(ctypes.c_int32 * 3)(4, 6, 8))),
    ("rope_dims 2", dict(rope_dims=2)),
    ("negative heads", dict(n_heads=-1)),
    ("theta zero", dict(rope_theta=0.0)),
    ("dtype", dict(dtype=7)),
    ("int4 with fp32", dict(cache_fmt=1)),
    ("int2 with fp32", dict(cache_fmt=2)),
    ("qk_norm flag", dict(qk_norm=2)),
    ("qk_norm eps negative", dict(qk_norm=1, qk_norm_eps=-1.0)),
    ("unknown cache format", dict(cache_fmt=3)),
]


@pytest.mark.parametrize("name,kw", BAD_DIMS, ids=[b[0] for b in BAD_DIMS])
def test_invalid_dims_rejected_before_launch(lib, name, kw):
    cfg = CONFIGS[1]
    d, g = _dims(cfg, **kw), _geom(cfg)
    fake = ctypes.c_void_p(0x1000)       # never dereferenced: validation fails first
    st = lib.mla_attention(ctypes.byref(d), ctypes.byref(g), None, 16, fake, fake, fake, fake, None,
                           fake, None, None, 0)
    assert st == _lib.MLA_ERR_INVALID_ARG, (name, st)
    assert lib.mla_last_error()


@pytest.mark.parametrize("fmt", [1, 2])
def test_lowbit_cache_needs_whole_groups(lib, fmt):
    cfg = SMALL_CONFIGS[5]              # bf16; a latent of 40 dims leaves a partial group of 32
    d, g = _dims(cfg, d_c=40, cache_fmt=fmt), _geom(cfg)
    fake = ctypes.c_void_p(0x1000)
    st = lib.mla_attention(ctypes.byref(d), ctypes.byref(g), None, 16, fake, fake, fake, fake, fake,
                           fake, None, None, 0)
    assert st == _lib.MLA_ERR_INVALID_ARG
    assert b"32" in lib.mla_last_error()


def test_invalid_geometry_and_pointers(lib):
    cfg = CONFIGS[3]
    d = _dims(cfg)
    fake = ctypes.c_void_p(0x1000)
    g = _geom(cfg, window=0)
    assert lib.mla_attention(ctypes.byref(d), ctypes.byref(g), None, 1, fake, fake, fake, fake, None,
                             fake, None, None, 0) == _lib.MLA_ERR_INVALID_ARG
    g = _geom(cfg)
    # NULL q_abs
    assert lib.mla_attention(ctypes.byref(d), ctypes.byref(g), None, 1, None, fake, fake, fake, None,
                             fake, None, None, 0) == _lib.MLA_ERR_INVALID_ARG
    assert b"q_abs" in lib.mla_last_error()
    # misaligned cache pointer
    assert lib.mla_attention(ctypes.byref(d), ctypes.byref(g), None, 1, fake, fake, fake,
                             ctypes.c_void_p(0x1002), None, fake, None, None, 0) == _lib.MLA_ERR_INVALID_ARG
    assert b"aligned" in lib.mla_last_error()
    # append: n_tokens not a whole number of frames
    assert lib.mla_cache_append(ctypes.byref(d), ctypes.byref(g), None, fake, 100, fake, fake, fake,
                                None, fake, 1 << 30) == _lib.MLA_ERR_INVALID_ARG
    assert b"multiple of P" in lib.mla_last_error()
    # append: more frames than the window
    assert lib.mla_cache_append(ctypes.byref(d), ctypes.byref(g), None, fake, 13 * 1560, fake, fake,
                                fake, None, fake, 1 << 40) == _lib.MLA_ERR_INVALID_ARG
    # append: workspace too small
    assert lib.mla_cache_append(ctypes.byref(d), ctypes.byref(g), None, fake, 1560, fake, fake, fake,
                                None, fake, 64) == _lib.MLA_ERR_WORKSPACE
    # INT4 cache needs the scale buffer
    d5, g5 = _dims(CONFIGS[5]), _geom(CONFIGS[5])
    assert lib.mla_attention(ctypes.byref(d5), ctypes.byref(g5), None, 1, fake, fake, fake, fake, None,
                             fake, None, fake, 1 << 40) == _lib.MLA_ERR_INVALID_ARG
    assert b"cache_aux" in lib.mla_last_error()


def test_zero_sizes_are_no_ops(lib):
    cfg = CONFIGS[3]
    d = _dims(cfg)
    g = _geom(cfg, batch=0)
    assert lib.mla_attention(ctypes.byref(d), ctypes.byref(g), None, 5, None, None, None, None, None,
                             None, None, None, 0) == _lib.MLA_OK
    g = _geom(cfg)
    assert lib.mla_absorb_q(ctypes.byref(d), ctypes.byref(g), None, 0, None, None, None, None,
                            None) == _lib.MLA_OK
    assert lib.mla_cache_append(ctypes.byref(d), ctypes.byref(g), None, None, 0, None, None, None,
                                None, None, 0) == _lib.MLA_OK


def test_unsupported_widths(lib):
    cfg = SMALL_CONFIGS[3]
    d = _dims(cfg, d_c=2048)
    g = _geom(cfg)
    fake = ctypes.c_void_p(0x1000)
    assert lib.mla_attention(ctypes.byref(d), ctypes.byref(g), None, 1, fake, fake, fake, fake, None,
                             fake, None, None, 0) == _lib.MLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("begin,count", [(-1, 4), (0, -1), (0, 10 ** 6), (5, 10 ** 6)])
def test_rope_shift_slot_range_rejected(lib, begin, count):
    cfg = SMALL_CONFIGS[3]
    d, g = _dims(cfg), _geom(cfg)
    fake = ctypes.c_void_p(0x1000)       # never dereferenced: validation fails first
    st = lib.mla_cache_rope_shift(ctypes.byref(d), ctypes.byref(g), None, fake, begin, count, fake, None)
    assert st == _lib.MLA_ERR_INVALID_ARG
    assert b"slots" in lib.mla_last_error()


def test_rope_shift_needs_aux_for_lowbit(lib):
    cfg = SMALL_CONFIGS[5]
    d, g = _dims(cfg), _geom(cfg)
    fake = ctypes.c_void_p(0x1000)
    st = lib.mla_cache_rope_shift(ctypes.byref(d), ctypes.byref(g), None, fake, 0, 4, fake, None)
    assert st == _lib.MLA_ERR_INVALID_ARG


@pytest.mark.parametrize("d_cq,status", [(0, _lib.MLA_ERR_INVALID_ARG), (-8, _lib.MLA_ERR_INVALID_ARG),
                                         (12, _lib.MLA_ERR_UNSUPPORTED)])
def test_query_fold_width_checked(lib, d_cq, status):
    cfg = SMALL_CONFIGS[3]                # bf16
    d, g = _dims(cfg), _geom(cfg)
    fake = ctypes.c_void_p(0x1000)
    assert lib.mla_fold_query_weights(ctypes.byref(d), None, d_cq, fake, fake, fake) == status
    assert lib.mla_absorb_q_folded(ctypes.byref(d), ctypes.byref(g), None, 4, d_cq, fake, fake, fake, fake,
                                   fake) == status
    assert lib.mla_last_error()


@pytest.mark.parametrize("key", [3, 5])
def test_qk_norm_aux_bytes(lib, key):
    cfg = CONFIGS[key]
    d, g = _dims(cfg), _geom(cfg)
    base = lib.mla_cache_aux_bytes(ctypes.byref(d), ctypes.byref(g))
    d.qk_norm, d.qk_norm_eps = 1, 1e-6
    na = lib.mla_cache_aux_bytes(ctypes.byref(d), ctypes.byref(g))
    rows = cfg.batch * cfg.capacity
    assert na == (base + 15) // 16 * 16 + 4 * rows


def test_qk_norm_entry_checks(lib):
    cfg = SMALL_CONFIGS[3]
    d, g = _dims(cfg), _geom(cfg)
    fake = ctypes.c_void_p(0x1000)
    # key norm without qk_norm set
    assert lib.mla_cache_key_norm(ctypes.byref(d), ctypes.byref(g), None, cfg.tokens_per_frame, fake, fake, fake,
                                  fake, None, 0) == _lib.MLA_ERR_INVALID_ARG
    d.qk_norm, d.qk_norm_eps = 1, 1e-6
    # a token count that is not a whole number of frames
    assert lib.mla_cache_key_norm(ctypes.byref(d), ctypes.byref(g), None, cfg.tokens_per_frame + 1, fake, fake,
                                  fake, fake, None, 0) == _lib.MLA_ERR_INVALID_ARG
    # a small call (one token per sequence) needs the partial-sum workspace
    dec = SMALL_CONFIGS[2]
    dd, gd = _dims(dec, qk_norm=1, qk_norm_eps=1e-6), _geom(dec)
    assert lib.mla_key_norm_workspace_size(ctypes.byref(dd), ctypes.byref(gd), 1) > 0
    assert lib.mla_cache_key_norm(ctypes.byref(dd), ctypes.byref(gd), None, 1, fake, fake, fake, fake, None,
                                  0) == _lib.MLA_ERR_WORKSPACE
    # the folded-query absorb has no query content values to normalise
    assert lib.mla_absorb_q_folded(ctypes.byref(d), ctypes.byref(g), None, 4, 64, fake, fake, fake, fake,
                                   fake) == _lib.MLA_ERR_UNSUPPORTED


def test_probe_argument_checks():
    """The measurement probes reject bad sizes and pointers before any launch."""
    lib = _lib.load_probe()
    inv = -1
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: the checks fail first
    assert lib.mla_probe_mfma(None, 0, 1, 0, fake, None) == inv
    assert lib.mla_probe_mfma(None, 1, 0, 0, fake, None) == inv
    assert lib.mla_probe_mfma(None, 1, 1, 2, fake, None) == inv
    assert lib.mla_probe_mfma(None, 1, 1, 1, None, None) == inv
    assert lib.mla_probe_hbm_read(None, fake, 0, 1, fake) == inv
    assert lib.mla_probe_hbm_read(None, fake, 24, 1, fake) == inv
    assert lib.mla_probe_hbm_read(None, fake, 32, 0, fake) == inv
    assert lib.mla_probe_hbm_read(None, None, 32, 1, fake) == inv
    assert lib.mla_probe_hbm_read(None, fake, 32, 1, ctypes.c_void_p(3)) == inv
    assert b"aligned" in lib.mla_probe_last_error()
