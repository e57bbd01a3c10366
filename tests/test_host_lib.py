"""CPU tests of libtq's host side: the library loads, exports every symbol
include/tq.h declares, its host table builder agrees with the oracle, and
invalid arguments are rejected before any GPU work (no compute calls here).
"""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

import kv_cache_vector_05_amd as tq
from kv_cache_vector_05_amd import _lib
from oracle import lloyd_max, rng as orng, rope as orope, rotation as orot

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(tq_[a-z_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 12, names
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert n in _lib.SIGNATURES, f"binding lacks {n}"
    L = tq.lib()
    for n in names:
        getattr(L, n)


def _ulps(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


@pytest.mark.parametrize("d", [64, 128, 1536])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_tables_match_oracle(d, bits):
    """Gauss-Legendre in C++ vs the incomplete beta function in the oracle:
    the float32 tables agree to within one unit in the last place."""
    m = 0
    rot = "dense" if d == 1536 else "hadamard"
    if rot == "dense":
        g = np.random.default_rng(0).standard_normal((d, d))
        t = tq.codebook_tables(d, bits, m, rot, rot_gauss=g)
    else:
        t = tq.codebook_tables(d, bits, m, rot, seed=1)
    lv, th = lloyd_max.table_f32(d, bits)
    assert _ulps(t["levels"], lv).max() <= 1
    assert _ulps(t["thresholds"], th).max() <= 1
    assert np.array_equal(t["levels"], -t["levels"][::-1]) and t["thresholds"][len(th) // 2] == 0


def test_seeded_draws_match_the_oracle_generator():
    """Both sides implement SplitMix64 + Box-Muller from their definitions."""
    d, m, seed = 128, 64, 12345
    t = tq.codebook_tables(d, 3, m, "hadamard", seed=seed)
    sigma, _, sketch = orng.seeded_draws(d, m, False, seed)
    np.testing.assert_array_equal(t["rotation"], sigma.astype(np.float32))
    assert _ulps(t["sketch"], sketch).max() <= 1


def test_seeded_dense_rotation_matches_oracle():
    d, seed = 64, 77
    t = tq.codebook_tables(d, 2, 32, "dense", seed=seed)
    _, g, _ = orng.seeded_draws(d, 32, True, seed)
    q = orot.haar_rotation(g)
    np.testing.assert_allclose(t["rotation"], q, atol=2e-7)
    r = t["rotation"].astype(np.float64)
    np.testing.assert_allclose(r @ r.T, np.eye(d), atol=1e-6)


def test_dense_rotation_from_given_draws():
    d = 256
    g = np.random.default_rng(3).standard_normal((d, d))
    t = tq.codebook_tables(d, 2, 0, "dense", rot_gauss=g)
    np.testing.assert_allclose(t["rotation"], orot.haar_rotation(g), atol=3e-7)


def test_given_draws_are_used_verbatim():
    d, m = 64, 32
    g = np.random.default_rng(4)
    sigma = np.where(g.integers(0, 2, d) == 1, 1, -1).astype(np.int8)
    sk = g.standard_normal((m, d)).astype(np.float32)
    t = tq.codebook_tables(d, 2, m, "hadamard", sigma=sigma, sketch=sk)
    np.testing.assert_array_equal(t["rotation"], sigma.astype(np.float32))
    np.testing.assert_array_equal(t["sketch"], sk)


def test_rope_table_matches_oracle():
    for base, d in [(500000.0, 128), (10000.0, 64)]:
        c, s = tq.rope_table(base, d, 4096, device=None)
        oc, os_ = orope.rope_table(base, d, 4096)
        assert _ulps(c, oc).max() <= 1 and _ulps(s, os_).max() <= 1


def test_plane_words():
    assert tq.plane_words(128, 3, 64) == (12, 2)
    assert tq.plane_words(128, 2, 128) == (8, 4)
    assert tq.plane_words(64, 3, 64) == (6, 2)
    assert tq.plane_words(1536, 2, 1536) == (96, 48)


@pytest.mark.parametrize("spec,code", [
    ((128, 0, 64, "auto"), _lib.TQ_EINVAL),       # bits 0
    ((128, 5, 64, "auto"), _lib.TQ_EINVAL),       # bits 5
    ((100, 3, 64, "auto"), _lib.TQ_EINVAL),       # bits*d not a multiple of 32
    ((128, 3, 48, "auto"), _lib.TQ_EINVAL),       # m not a multiple of 32
    ((96, 2, 0, "hadamard"), _lib.TQ_EINVAL),     # Hadamard needs a power of two
    ((256, 2, 0, "hadamard"), _lib.TQ_EUNSUPPORTED),
    ((128, 2, 96, "hadamard"), _lib.TQ_EUNSUPPORTED),
    ((96, 2, 0, "dense"), _lib.TQ_EUNSUPPORTED),  # dense needs a multiple of 64
])
def test_bad_specs_are_rejected(spec, code):
    d, bits, m, rot = spec
    with pytest.raises(tq.TQError) as ei:
        tq.codebook_tables(d, bits, m, rot)
    assert ei.value.code == code
    assert tq.lib().tq_last_error().decode()


def test_null_arguments_are_rejected_without_a_gpu():
    L = tq.lib()
    assert L.tq_codebook_init(None, None, None, None) == _lib.TQ_EINVAL
    h = C.c_void_p()
    assert L.tq_codebook_init(None, None, None, C.byref(h)) == _lib.TQ_EINVAL and not h.value
    assert L.tq_codebook_destroy(None) == _lib.TQ_OK
    assert L.tq_encode_kv(None, None, None, None, 0, 1, 1, 1, None, None, 0, 1, None, None, 0, None, None, None,
                          0, None) == _lib.TQ_EINVAL
    assert L.tq_attn_logits(None, None, 0, None, 1, 1, 1, 1, None, None, None, None, 0, 0, None, None, None, 0,
                            None) == _lib.TQ_EINVAL
    assert L.tq_attn_decode(None, None, None, 0, None, None, 1, 1, 1, 1, None, None, None, None, 0, 0.0, None, None,
                            0, None) == _lib.TQ_EINVAL
    assert L.tq_rope_table(10000.0, 63, 4, None, None) == _lib.TQ_EINVAL
    assert L.tq_workspace_bytes(None, None, 0, 10, 1, 1, 1, 0) == 0
    assert L.tq_version().decode().startswith("libtq")


def test_forced_allocation_failure_reports_enomem(monkeypatch):
    monkeypatch.setenv("TQ_TEST_FAIL_ALLOC", "1")
    sp = _lib.tq_spec(64, 2, 32, 0, 0)
    h = C.c_void_p()
    assert tq.lib().tq_codebook_init(C.byref(sp), None, None, C.byref(h)) == _lib.TQ_ENOMEM
    assert not h.value


def test_paged_and_append_calls_reject_bad_arguments_without_a_gpu():
    """Page tables and appends are checked on the host before any launch."""
    L = tq.lib()
    sp = _lib.tq_spec(64, 2, 32, 0, 0)
    for size, maxp, npg in [(48, 4, 8), (0, 4, 8), (64, 0, 8), (64, 4, 0), (64, 1 << 25, 8)]:
        pg = _lib.tq_pages(1, size, maxp, npg)
        assert L.tq_attn_logits_paged(None, None, 0, None, 1, 1, 1, None, None, C.byref(pg), None, None, 0, 0,
                                      None, None, None, 0, None) == _lib.TQ_EINVAL
    pg = _lib.tq_pages(None, 64, 4, 8)
    assert L.tq_attn_decode_paged(None, None, None, 0, None, None, 1, 1, 1, None, None, C.byref(pg), None, None, 0,
                                  0.0, None, None, 0, None) == _lib.TQ_EINVAL
    assert L.tq_encode_kv_paged(None, None, None, None, 0, 1, 1, 1, None, None, 0, None, None, None, 0, None, None,
                                None) == _lib.TQ_EINVAL
    # append: no positions, or no page table and no capacity
    assert L.tq_append_kv(None, None, None, None, 0, 1, 1, None, None, None, None, 8, None, None, 0, None, None,
                          None) == _lib.TQ_EINVAL
    assert L.tq_append_kv(None, None, None, None, 0, 1, 1, None, None, C.c_void_p(16), None, 0, None, None, 0, None,
                          None, None) == _lib.TQ_EINVAL


def test_missing_library_fails_loudly(tmp_path):
    """Without the built library every call raises: the binding has no other
    path to fall back on."""
    import sys
    code = ("import kv_cache_vector_05_amd as tq\n"
            "try:\n"
            "    tq.Codebook(64, 2, 0, 'hadamard', seed=1)\n"
            "except ImportError as e:\n"
            "    print('RAISED', e)\n")
    env = dict(os.environ, TQ_LIBRARY=str(tmp_path / "absent" / "libtq.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    assert "RAISED" in r.stdout and "not built" in r.stdout, r.stdout
