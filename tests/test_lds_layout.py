"""The LDS tile layout shared by the chunked prefill and the prefix-aware decode (csrc/lds_tile.hpp),
checked on the CPU for every lane and operand read: a host program built from the header prints
its XOR swizzles, and this test replays the DMA writes and the MFMA operand reads of both kernels.

- Every 16-byte chunk of every K row and V row lands in exactly one LDS slot of its row, and the
  read of source chunk x of a row finds it there (the layout is a bijection, read back exactly).
- The sixteen lanes that one 128-bit LDS read serves together (lanes 16i .. 16i+15) hit sixteen
  different 16-byte bank groups of the 64 x 4-byte banks, for every K and V operand read.
"""
import os
import subprocess

import pytest

from paged_kv_cache_190_amd import build as b

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "paged_kv_cache_190_amd", "csrc")


@pytest.fixture(scope="module")
def swizzles(tmp_path_factory):
    d = tmp_path_factory.mktemp("lds")
    src = d / "tables.hip"
    src.write_text('#include "lds_tile.hpp"\n#include <cstdio>\nint main() {\n'
                   '  for (int r = 0; r < 32; ++r) std::printf("k128 %d %d\\n", r, pkv::kswz<128>(r));\n'
                   '  for (int r = 0; r < 32; ++r) std::printf("k64 %d %d\\n", r, pkv::kswz<64>(r));\n'
                   '  for (int r = 0; r < 128; ++r) std::printf("v %d %d\\n", r, pkv::vswz(r));\n'
                   '  return 0;\n}\n')
    exe = d / "tables"
    r = subprocess.run([b.hipcc(), "-O1", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    t = {"k128": {}, "k64": {}, "v": {}}
    for line in out.split("\n"):
        if line:
            k, row, x = line.split()
            t[k][int(row)] = int(x)
    return t


def krow_of(col):
    # MFMA row of the K operand for lane column col (lane half hb then picks chunks 2kk + hb)
    return 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3)


@pytest.mark.parametrize("D", [64, 128])
def test_k_tile_layout(swizzles, D):
    kswz = swizzles[f"k{D}"]
    cpr = D // 8            # 16-byte chunks per K row
    krow_bytes = 2 * D
    # DMA side: instruction c, lane l writes LDS slot (c KiB + 16 l) with source chunk
    # (l % cpr) ^ kswz(row) of row c * (64 / cpr) + l / cpr
    holds = {}
    for c in range(32 * krow_bytes // 1024):
        for lane in range(64):
            prow = c * (64 // cpr) + lane // cpr
            chunk = (lane % cpr) ^ kswz[prow]
            slot = c * 1024 + 16 * lane
            assert slot == prow * krow_bytes + 16 * (lane % cpr)
            holds[slot] = (prow, chunk)
    assert sorted(holds.values()) == [(r, x) for r in range(32) for x in range(cpr)]
    # read side: lane (col, hb) reads source chunk 2 kk + hb of row krow(col)
    for kk in range(D // 16):
        banks = {}
        for lane in range(64):
            col, hb = lane & 31, lane >> 5
            row = krow_of(col)
            want = 2 * kk + hb
            addr = row * krow_bytes + 16 * (want ^ kswz[row])
            assert holds[addr] == (row, want)
            banks.setdefault(lane // 16, []).append((addr // 16) % 16)
        for group, g in banks.items():
            assert len(set(g)) == 16, f"D={D} kk={kk} lanes {16 * group}..: bank groups {g}"


@pytest.mark.parametrize("D", [64, 128])
def test_v_tile_layout(swizzles, D):
    vswz = swizzles["v"]
    k_bytes = 32 * 2 * D
    # DMA side: V instruction c, lane l: dim d = c * 16 + l / 4, slot chunk l & 3 holds source
    # chunk (keys 8 x .. 8 x + 7) x = (l & 3) ^ vswz(d); rows of 64 bytes after the K tile
    holds = {}
    for c in range(D * 64 // 1024):
        for lane in range(64):
            d = c * 16 + lane // 4
            chunk = (lane & 3) ^ vswz[d]
            slot = k_bytes + c * 1024 + 16 * lane
            assert slot == k_bytes + d * 64 + 16 * (lane & 3)
            holds[slot] = (d, chunk)
    assert sorted(holds.values()) == [(d, x) for d in range(D) for x in range(4)]
    # read side: lane (col, hb) reads keys 16 hb + 8 j .. of dim 32 dt + col, j = 0, 1
    for dt in range(D // 32):
        for j in range(2):
            banks = {}
            for lane in range(64):
                col, hb = lane & 31, lane >> 5
                d = 32 * dt + col
                want = 2 * hb + j
                addr = k_bytes + d * 64 + 16 * (want ^ vswz[col])
                assert holds[addr] == (d, want)
                banks.setdefault(lane // 16, []).append((addr // 16) % 16)
            for group, g in banks.items():
                assert len(set(g)) == 16, f"D={D} dt={dt} j={j} lanes {16 * group}..: {g}"
