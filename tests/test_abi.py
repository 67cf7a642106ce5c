"""The C ABI library: it loads, exports every declared symbol, and its host-only
functions agree with the oracle (no GPU needed)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from paged_decode_attention_tq_amd import _lib, api
from tests.conftest import ROOT


def _declared():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "tq_write_kv" in names and "tq_paged_decode" in names
    lib = _lib.lib()
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_row_bytes():
    for bits, rb in ((2, 36), (3, 52), (4, 68), (5, 84)):
        assert api.row_bytes(128, bits) == rb == oracle.row_bytes(128, bits)
    assert api.row_bytes(0, 4) == 0 and api.row_bytes(128, 9) == 0


@pytest.mark.parametrize("d", [3, 4, 16, 64, 128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_host_codebook_equals_oracle(d, bits):
    # two independent solvers (long-double recursion vs scipy/mpmath) agree bit for bit
    c, t = api.codebook(d, bits)
    _, c32, t64 = oracle.beta_codebook(d, bits)
    assert np.array_equal(c, c32)
    assert np.array_equal(t, t64.astype(np.float32))


@pytest.mark.parametrize("seed", [0, 42, 7, 2**63 + 5])
def test_host_signs_equal_oracle(seed):
    assert np.array_equal(api.rht_signs(seed, 256), oracle.rht_signs(seed, 256))


def test_status_strings_and_argument_errors():
    lib = _lib.lib()
    assert lib.tq_status_string(0) == b"ok"
    assert lib.tq_status_string(4) == b"workspace too small"
    ctx = api.Context(128, 42)
    h = ctx.handle
    # these fail validation before any HIP call
    assert lib.tq_write_kv(h, None, 1, 4, 2, None, 4, 16, None, 7, None, None) == 2  # bits 7
    assert lib.tq_write_kv(h, None, 1, 4, 2, None, 4, 16, None, 4, None, None) == 1  # null raw
    assert lib.tq_write_kv(h, None, 9, 4, 2, None, 4, 16, None, 4, None, None) == 1  # bad dtype
    assert lib.tq_write_kv(h, None, 1, 0, 2, None, 4, 16, None, 4, None, None) == 0  # nothing to do
    # the K+V pair: each component's arguments are checked the same way
    pw = lib.tq_write_kv_pair
    a64 = ctypes.c_void_p(64)  # aligned, never dereferenced: validation fails first
    assert pw(h, a64, a64, 1, 4, 2, a64, 4, a64, 7, 4, 16, a64, None, None) == 2  # V bits 7
    assert pw(h, None, None, 1, 4, 2, None, 9, None, 4, 4, 16, None, None, None) == 2  # K bits 9
    assert pw(h, None, None, 1, 4, 2, None, 4, None, 4, 4, 16, None, None, None) == 1  # null pointers
    assert pw(h, None, None, 1, 0, 2, None, 4, None, 2, 4, 16, None, None, None) == 0  # nothing to do
    assert pw(h, ctypes.c_void_p(64), ctypes.c_void_p(66), 1, 4, 2, ctypes.c_void_p(64), 4,
              ctypes.c_void_p(64), 4, 4, 16, ctypes.c_void_p(64), None, None) == 3  # raw_v misaligned
    # the dense readback
    rd = lib.tq_decompress_kv
    assert rd(h, a64, 4, 16, 2, 6, a64, 5, a64, 0, None, None) == 2  # bits 6
    assert rd(h, a64, 4, 16, 2, 4, a64, 5, a64, 7, None, None) == 1  # bad out dtype
    assert rd(h, None, 4, 16, 2, 4, a64, 5, a64, 0, None, None) == 1  # null pages
    assert rd(h, a64, 4, 16, 0, 4, a64, 5, a64, 0, None, None) == 1  # no KV heads
    assert rd(h, a64, 4, 16, 2, 4, a64, 0, None, 0, None, None) == 0  # nothing to read
    assert rd(h, a64, 4, 16, 2, 4, ctypes.c_void_p(68), 5, a64, 0, None, None) == 3  # slots not 8-byte aligned
    assert rd(h, a64, 4, 16, 2, 4, a64, 5, ctypes.c_void_p(72), 0, None, None) == 3  # out not 16-byte aligned
    assert rd(h, a64, 4, 16, 2, 4, a64, 1 << 30, a64, 0, None, None) == 2  # 2^31 rows
    # the hybrid decode: its own checks, then the decode's
    hy = lib.tq_paged_decode_hybrid
    p = ctypes.c_void_p(16)
    need = lib.tq_hybrid_workspace_bytes(h, 2, 8, 2, 64, 16)
    assert need >= lib.tq_decode_workspace_bytes(h, 2, 8, 2, 64, 16) + 2 * 8 * 4
    assert hy(h, p, 1, 2, 8, 2, p, 4, p, 4, 8, 16, p, 4, p, 64, p, p, 7, 16, p, 0.0, p, p, need, None) == 1  # dtype
    assert hy(h, p, 1, 2, 8, 2, p, 4, p, 4, 8, 16, p, 4, p, 64, None, p, 1, 16, p, 0.0, p, p, need, None) == 1  # null window
    assert hy(h, p, 1, 2, 8, 2, p, 4, p, 4, 8, 16, p, 4, p, 64, ctypes.c_void_p(24), p, 1, 16, p, 0.0, p, p, need,
              None) == 3  # window not 16-byte aligned
    assert hy(h, p, 1, 2, 8, 2, p, 4, p, 4, 8, 16, p, 4, p, 64, p, p, 1, 16, p, 0.0, p, p, need - 4, None) == 4
    assert hy(h, p, 1, 2, 8, 2, p, 4, p, 4, 8, 16, p, 4, p, 64, p, p, 1, -1, p, 0.0, p, p, need, None) == 1  # cap < 0
    assert hy(h, p, 1, 2, 8, 2, p, 4, p, 4, 8, 32, p, 4, p, 64, p, p, 1, 16, p, 0.0, p, p, need, None) == 2  # block 32
    # the one-call decode step: its own checks, then the decode's
    ap = lib.tq_paged_decode_append
    dneed = lib.tq_decode_workspace_bytes(h, 2, 8, 2, 64, 16)
    assert ap(h, p, 1, 2, 8, 2, p, p, 7, p, 4, p, 4, 8, 16, p, 4, p, 64, 0.0, p, p, dneed, None, None) == 1  # row dtype
    assert ap(h, p, 1, 2, 8, 2, None, p, 1, p, 4, p, 4, 8, 16, p, 4, p, 64, 0.0, p, p, dneed, None, None) == 1  # no k_new
    assert ap(h, p, 1, 2, 8, 2, p, ctypes.c_void_p(18), 1, p, 4, p, 4, 8, 16, p, 4, p, 64, 0.0, p, p, dneed, None,
              None) == 3  # v_new misaligned
    assert ap(h, p, 1, 2, 8, 2, p, p, 1, p, 6, p, 4, 8, 16, p, 4, p, 64, 0.0, p, p, dneed, None, None) == 2  # K bits 6
    assert ap(h, p, 1, 2, 8, 2, p, p, 1, p, 4, p, 4, 8, 16, p, 4, p, 64, 0.0, p, p, dneed - 4, None, None) == 4
    assert ap(h, p, 1, 0, 8, 2, None, None, 1, p, 4, p, 4, 8, 16, p, 4, p, 64, 0.0, p, p, dneed, None, None) == 0
    # the prod key codec
    assert [lib.tq_prod_row_bytes(128, b) for b in (2, 3, 4, 5)] == [40, 56, 72, 88]
    assert lib.tq_prod_row_bytes(128, 1) == 0 and lib.tq_prod_row_bytes(100, 4) == 0
    wp = lib.tq_write_kv_prod
    assert wp(h, a64, 1, 4, 2, a64, 4, 16, a64, 6, a64, None, None) == 2  # bits 6
    assert wp(h, a64, 1, 4, 2, a64, 4, 16, a64, 4, None, None, None) == 1  # no sketch
    assert wp(h, a64, 1, 4, 2, a64, 4, 16, a64, 4, ctypes.c_void_p(68), None, None) == 3  # sketch alignment
    assert wp(h, a64, 1, 0, 2, a64, 4, 16, a64, 4, None, None, None) == 0  # nothing to write
    ps = lib.tq_prod_scores
    wsb = lib.tq_prod_scores_workspace_bytes(2, 8)
    assert wsb == 2 * 2 * 8 * 128 * 4
    assert ps(h, a64, 1, 2, 8, 2, a64, 4, 8, 16, a64, 4, a64, 64, a64, a64, a64, wsb - 4, None) == 4
    assert ps(h, a64, 1, 2, 8, 2, a64, 7, 8, 16, a64, 4, a64, 64, a64, a64, a64, wsb, None) == 2  # bits 7
    assert ps(h, a64, 1, 2, 8, 2, a64, 4, 8, 16, a64, 4, a64, 64, None, a64, a64, wsb, None) == 1  # no sketch
    assert ps(h, a64, 1, 2, 8, 3, a64, 4, 8, 16, a64, 4, a64, 64, a64, a64, a64, wsb, None) == 1  # 8 % 3
    assert ps(h, a64, 1, 2, 8, 2, a64, 4, 8, 16, a64, 1 << 22, a64, 1 << 26, a64, a64, a64, wsb,
              None) == 2  # 2^26 score columns
    # multi-query attention
    pf = lib.tq_paged_prefill
    a256 = ctypes.c_void_p(256)
    need = lib.tq_prefill_workspace_bytes(h, 2, 4, 16, 2, 64, 16)
    assert need > lib.tq_hybrid_workspace_bytes(h, 2, 64, 2, 64, 16)
    assert pf(h, a256, 1, 2, 9, a256, 16, 2, a256, 4, a256, 4, 8, 16, a256, 4, a256, 64, 0.0, a256, a256, need,
              None) == 2  # 8 query heads x 9 queries > 64
    assert pf(h, a256, 1, 2, 0, a256, 16, 2, a256, 4, a256, 4, 8, 16, a256, 4, a256, 64, 0.0, a256, a256, need,
              None) == 1  # q_len 0
    assert pf(h, ctypes.c_void_p(260), 1, 2, 4, a256, 16, 2, a256, 4, a256, 4, 8, 16, a256, 4, a256, 64, 0.0, a256,
              a256, need, None) == 3  # q not 16-byte aligned
    assert pf(h, a256, 1, 2, 4, a256, 16, 2, a256, 4, a256, 4, 8, 16, a256, 4, a256, 64, 0.0, a256,
              ctypes.c_void_p(272), need, None) == 3  # workspace not 256-byte aligned
    assert pf(h, a256, 1, 2, 4, a256, 16, 2, a256, 4, a256, 4, 8, 16, a256, 4, a256, 64, 0.0, a256, a256, need - 1,
              None) == 4
    assert pf(h, a256, 1, 2, 4, None, 16, 2, a256, 4, a256, 4, 8, 16, a256, 4, a256, 64, 0.0, a256, a256, need,
              None) == 1  # no q_lens
    args = dict(batch=2, hq=128, hkv=1)  # group 128 > 64
    assert lib.tq_paged_decode(h, p, 1, 2, 128, 1, p, 4, p, 4, 8, 16, p, 4, p, 64, 0.0, p, p, 1 << 20, None) == 2
    assert lib.tq_paged_decode(h, p, 1, 2, 6, 4, p, 4, p, 4, 8, 16, p, 4, p, 64, 0.0, p, p, 1 << 20, None) == 1
    assert lib.tq_paged_decode(h, p, 1, 2, 8, 2, p, 4, p, 4, 8, 32, p, 4, p, 64, 0.0, p, p, 1 << 20, None) == 2
    assert lib.tq_paged_decode(h, p, 1, 2, 8, 2, p, 4, p, 4, 8, 16, p, 4, p, 64, 0.0, p, p, 16, None) == 4
    assert lib.tq_paged_decode(h, p, 1, 2, 8, 2, p, 4, p, 4, 8, 16, p, 3, p, 64, 0.0, p, p, 1 << 20, None) == 1
    odd = ctypes.c_void_p(18)
    assert lib.tq_paged_decode(h, p, 1, 2, 8, 2, odd, 4, p, 4, 8, 16, p, 4, p, 64, 0.0, p, p, 1 << 20, None) == 3
    with pytest.raises(ValueError):
        _lib.check(2, "x")
    with pytest.raises(_lib.TQError):
        _lib.check(4, "x")
    del args


def test_context_rejects_other_head_dims():
    with pytest.raises(ValueError):
        api.Context(64, 42)


def test_decode_kernel_choice():
    # host-only planning (no device: the compute-unit count defaults to 256)
    assert api.decode_kernel(1, 2, 1, 64, 4, 4) == "wave1"          # 4 pages: one workgroup, no merge kernel
    assert api.decode_kernel(8, 16, 2, 64, 4, 4) == "wave1"         # 32 pages
    assert api.decode_kernel(3, 16, 2, 200, 4, 4) == "wave"         # 39 pages: split over workgroups
    assert api.decode_kernel(65, 16, 2, 16, 4, 4) == "wave"         # more than 64 sequences
    assert api.decode_kernel(32, 16, 2, 2048, 4, 4) == "wave"       # pages geometry
    assert api.decode_kernel(8, 64, 8, 131072, 4, 4) == "staged"    # 8 KV heads
    assert api.decode_kernel(2, 16, 1, 64, 4, 4) == "staged"        # 16 query heads per KV head
    assert api.decode_kernel(2, 16, 3, 64, 4, 4) is None            # 16 % 3 != 0
    assert api.decode_kernel(2, 8, 2, 64, 7, 4) is None             # 7 bits
