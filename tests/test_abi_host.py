"""Host-side checks of the C-ABI library that need no GPU.

* The shared library loads and exports every function declared in include/*.h.
* bsl_block_bytes agrees with the printed block size (7.56 MB) and the oracle's formula.
* The host packer ("bitstack_pack") follows the documented tile layout bit by bit, and
  bsl_unpack_signs inverts it; both are compared with the oracle's own row-major signs.
* Argument validation returns the documented error codes without touching a device.
"""
from __future__ import annotations

import glob
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

bsl = pytest.importorskip("bit_sign_rank_amd")
if not os.path.exists(bsl.LIB_PATH):
    pytest.skip("libbitstack_linear.so not built", allow_module_level=True)


def _declared_functions():
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(bsl_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert len(declared) >= 14
    L = bsl.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) == set(bsl.EXPORTED)


def test_binding_constants_match_the_header():
    defines = {}
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        for name, value in re.findall(r"^#define (BSL_[A-Z0-9_]+) \(?(-?\d+)\)?", open(path).read(), flags=re.M):
            defines[name] = int(value)
    assert {"BSL_PATH_AUTO", "BSL_PATH_DECODE", "BSL_PATH_PRODUCT", "BSL_KERNEL_KINDS"} <= set(defines)
    for name, value in defines.items():
        assert getattr(bsl, name) == value, name


@pytest.mark.parametrize("m,d", [(14336, 4096), (4096, 14336), (1024, 1024), (8, 8), (11008, 4096)])
def test_block_bytes(m, d):
    assert bsl.bsl_block_bytes(m, d, 16) == oracle.block_bytes(m, d, 16)


def test_block_bytes_printed_value():
    assert round(bsl.bsl_block_bytes(14336, 4096, 16) / 2**20, 2) == 7.56


def _expected_tiled(bits, m, d):
    """The documented layout, written out independently of the library: tiles ordered
    [column chunk c][row tile t], rows padded to 1024; in tile (c, t), bit p of word q of
    lane 16 g + i is the sign of row 16 t + i, column 512 c + 32 b + 8 g + e with
    e = (p % 16) // 2, b = 4 q + k, k = p // 16 + (0 if p is odd else 2) (padding reads
    as +1, i.e. bit 0)."""
    signs_neg = np.unpackbits(bits, axis=1, bitorder="little")[:, :d].astype(np.uint8)
    mp = -(-m // 1024) * 1024  # rows padded to 1024
    dp = -(-d // 512) * 512
    full = np.zeros((mp, dp), np.uint8)
    full[:m, :d] = signs_neg
    nch = dp // 512
    out = np.zeros((nch, mp // 16, 64, 4), np.uint32)  # [chunk][row tile][lane][word]
    p = np.arange(32)
    k = p // 16 + np.where(p % 2 == 1, 0, 2)
    e = (p % 16) // 2
    for g in range(4):
        for q in range(4):
            cols = 32 * (4 * q + k) + 8 * g + e
            for c in range(nch):
                blk = full[:, 512 * c + cols].reshape(mp // 16, 16, 32).astype(np.uint64)
                words = (blk << p.astype(np.uint64)).sum(axis=2).astype(np.uint32)
                for i in range(16):
                    out[c, :, 16 * g + i, q] = words[:, i]
    return out.view(np.uint8).reshape(-1)


@pytest.mark.parametrize("m,d", [(16, 512), (48, 1536), (37, 520), (5, 8), (64, 4096)])
def test_pack_layout_matches_spec(m, d):
    bits = synth.sign_bits(31, m, d, m, d)
    tiled = bsl.bsl_pack_signs(bits, m, d)
    assert tiled.size == bsl.bsl_packed_sign_bytes(m, d)
    assert np.array_equal(tiled, _expected_tiled(bits, m, d))


@pytest.mark.parametrize("m,d", [(16, 512), (33, 1032), (128, 2048), (3, 24)])
def test_pack_unpack_round_trip_matches_oracle(m, d):
    bits = synth.sign_bits(7, m, d, m, d)
    tiled = bsl.bsl_pack_signs(bits, m, d)
    assert np.array_equal(bsl.bsl_unpack_signs(tiled, m, d), oracle.signs_from_bits(bits, d))


@pytest.mark.parametrize("pattern", ["plus", "minus", "checker", "edges"])
def test_pack_adversarial_patterns(pattern):
    m, d = 32, 1024
    s = np.ones((m, d), np.int8)
    if pattern == "minus":
        s[:] = -1
    elif pattern == "checker":
        s[(np.arange(m)[:, None] + np.arange(d)[None, :]) % 2 == 1] = -1
    elif pattern == "edges":
        for c in (0, 7, 8, 31, 32, 255, 256, 511, 512, 1023):
            s[(c * 7) % m, c] = -1
        s[15, :] = -1
        s[16, 511] = -1
    bits = oracle.bits_from_signs(s)
    tiled = bsl.bsl_pack_signs(bits, m, d)
    assert np.array_equal(tiled, _expected_tiled(bits, m, d))
    assert np.array_equal(bsl.bsl_unpack_signs(tiled, m, d), s)


def test_pack_rejects_bad_shapes():
    with pytest.raises(bsl.BslError) as e:
        bsl.bsl_pack_signs(np.zeros(0, np.uint8), 4, 4)
    assert e.value.code == bsl.BSL_EUNSUPPORTED


def test_init_validates_before_touching_a_device():
    with pytest.raises(bsl.BslError) as e:
        bsl.bsl_init(0, [64], [512], k=8)
    assert e.value.code == bsl.BSL_EUNSUPPORTED
    with pytest.raises(bsl.BslError) as e:
        bsl.bsl_init(0, [64], [100])
    assert e.value.code == bsl.BSL_EUNSUPPORTED
    with pytest.raises(bsl.BslError) as e:
        bsl.bsl_init(0, [64], [512], n_cap=0)
    assert e.value.code == bsl.BSL_EINVAL


def test_lowrank_init_validates_before_touching_a_device():
    for m, d, kp, n_cap, code in [([64], [100], [8], 4, bsl.BSL_EUNSUPPORTED), ([64], [512], [0], 4, bsl.BSL_EUNSUPPORTED),
                                  ([64], [512], [2000], 4, bsl.BSL_EUNSUPPORTED), ([64], [512], [8], 0, bsl.BSL_EINVAL)]:
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_lr_init(0, m, d, kp, n_cap)
        assert e.value.code == code


@pytest.mark.parametrize("m,d", [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336), (8192, 28672), (37, 520)])
def test_lowrank_sizes_match_the_oracle(m, d):
    kp = bsl.bsl_lr_equal_rank(m, d, 16)
    assert kp == oracle.equal_bytes_rank(m, d, 16)
    assert bsl.bsl_lr_block_bytes(m, d, kp) == oracle.lowrank_block_bytes(m, d, kp)
