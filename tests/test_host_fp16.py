"""The library's host-side binary16 conversions (used to fold an input-channel scale
into V at load), compiled alone with the host C++ compiler and compared with numpy's
IEEE conversions: every fp16 bit pattern to double, and doubles to fp16 with ties to
even at every halfway point, around the subnormal and overflow boundaries, and at
random."""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_sign_rank_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <vector>
#include "bsl_fp16.h"
int main(int argc, char** argv) {
  // argv[1]: doubles in; argv[2]: [fp16 bits, ok] pairs out; argv[3]: all 65536 fp16 -> double
  FILE* f = std::fopen(argv[1], "rb");
  std::vector<double> v;
  double t;
  while (std::fread(&t, 8, 1, f) == 1) v.push_back(t);
  std::fclose(f);
  std::vector<uint16_t> out(2 * v.size());
  for (size_t i = 0; i < v.size(); ++i) out[2 * i + 1] = bsl::double_to_fp16(v[i], &out[2 * i]) ? 1 : 0;
  f = std::fopen(argv[2], "wb");
  std::fwrite(out.data(), 2, out.size(), f);
  std::fclose(f);
  std::vector<double> back(65536);
  for (uint32_t h = 0; h < 65536; ++h) back[h] = bsl::fp16_to_double((uint16_t)h);
  f = std::fopen(argv[3], "wb");
  std::fwrite(back.data(), 8, back.size(), f);
  std::fclose(f);
  return 0;
}
"""


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("fp16")
    src = d / "drv.cpp"
    src.write_text(DRIVER)
    exe = d / "drv"
    subprocess.run([cxx, "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    return d, exe


def _run(driver, vals):
    d, exe = driver
    vals = np.ascontiguousarray(vals, dtype=np.float64)
    (d / "in.bin").write_bytes(vals.tobytes())
    subprocess.run([str(exe), str(d / "in.bin"), str(d / "out.bin"), str(d / "back.bin")], check=True)
    out = np.fromfile(d / "out.bin", dtype=np.uint16).reshape(-1, 2)
    back = np.fromfile(d / "back.bin", dtype=np.float64)
    return out[:, 0], out[:, 1].astype(bool), back


def _test_values():
    all16 = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    fin = np.unique(all16[np.isfinite(all16)])
    pos = fin[fin >= 0]
    mids = (pos[:-1] + pos[1:]) / 2  # exact halfway points (ties)
    nudge = np.concatenate([mids * (1 + 2.0**-40), mids * (1 - 2.0**-40)])
    g = np.random.default_rng(5)
    rnd = np.ldexp(g.uniform(0.5, 1.0, 20000), g.integers(-30, 18, 20000))
    edges = np.array([0.0, 2.0**-25, 2.0**-25 * 1.0000001, 2.0**-24, 1.5 * 2.0**-24, 2.0**-14, 2.0**-14 * (1 - 2.0**-12),
                      65504.0, 65519.999, 65520.0, 65536.0, 1e300, 5e-324, 1e-310])
    v = np.concatenate([pos, mids, nudge, rnd, edges])
    return np.concatenate([v, -v, [np.inf, -np.inf, np.nan]])


def test_fp16_bits_to_double_matches_ieee(driver):
    _, _, back = _run(driver, np.zeros(1))
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(back), nan)
    assert np.array_equal(back[~nan], ref[~nan])
    assert np.array_equal(np.signbit(back[~nan]), np.signbit(ref[~nan]))


def test_double_to_fp16_rounds_to_nearest_even(driver):
    v = _test_values()
    bits, ok, _ = _run(driver, v)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = v.astype(np.float16)
    finite = np.isfinite(ref)
    assert np.array_equal(ok, finite)  # overflow and non-finite inputs are refused
    assert np.array_equal(bits[finite], ref[finite].view(np.uint16))
