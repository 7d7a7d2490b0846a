"""Host-side check of the LDS tile layout the attention kernels use.

tests/lds_layout_dump.cpp prints the offsets computed by the kernels' own
layout header (exact_attention_84_amd/csrc/fa_layout.hpp).  This test fills a
model of a 64-key tile the way the direct global->LDS loads do, replays every
MFMA operand read the kernels issue, and checks (1) that each lane receives
exactly the K / V values its MFMA operand slot needs and (2) that no read has
an LDS bank conflict, modelling gfx950's LDS as 64 banks of 4 bytes that serve
16 lanes per clock for 16-byte reads and 32 lanes per clock for 8-byte reads.
The transposing read (ds_read_b64_tr_b16) is modelled as measured on the GPU:
within each group of 16 lanes, result lane i element j is element i & 3 of the
8 bytes addressed by source lane 4 j + (i >> 2).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "lds_layout_dump.cpp")
INC = os.path.join(ROOT, "exact_attention_84_amd", "csrc")
BC = 64  # keys per tile


@pytest.fixture(scope="module")
def dump(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("lds") / "dump")
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", INC, SRC, "-o", exe], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    tables, cur = {}, None
    for line in out.splitlines():
        f = line.split()
        if f[0] == "D":
            cur = tables.setdefault(int(f[1]), {"dma": {}, "k": {}, "v": {}})
        elif f[0] == "dma":
            cur["dma"][(int(f[1]), int(f[2]))] = (int(f[3]), int(f[4]))
        elif f[0] == "k":
            cur["k"][(int(f[1]), int(f[2]))] = int(f[3])
        else:
            cur["v"][(int(f[1]), int(f[2]), int(f[3]))] = int(f[4])
    return tables


def fill_tile(d, tab):
    """Element ids (key * d + column) at each 2-byte LDS slot after the fill."""
    vals = np.arange(BC * d).reshape(BC, d)
    lds = np.full(BC * d, -1)
    for (inst, lane), (row, chunk) in tab["dma"].items():
        dst = (inst * 1024 + lane * 16) // 2
        lds[dst:dst + 8] = vals[row, chunk * 8:chunk * 8 + 8]
    return vals, lds


def conflict_cycles(addrs, lanes_per_clock, words):
    extra = 0
    for g in range(0, 64, lanes_per_clock):
        hits = {}
        for a in addrs[g:g + lanes_per_clock]:
            for w in range(words):
                b = (a // 4 + w) % 64
                hits[b] = hits.get(b, 0) + 1
        extra += max(hits.values()) - 1
    return extra


@pytest.mark.parametrize("d", [128, 64])
def test_tile_fill_covers_every_element_once(dump, d):
    _, lds = fill_tile(d, dump[d])
    assert (lds >= 0).all()
    assert len(np.unique(lds)) == lds.size


@pytest.mark.parametrize("d", [128, 64])
def test_k_operand_reads(dump, d):
    vals, lds = fill_tile(d, dump[d])
    tab = dump[d]
    for kt in range(BC // 32):
        for st in range(d // 16):
            addrs = [tab["k"][(st, lane)] + kt * 64 * d for lane in range(64)]
            for lane in range(64):
                got = lds[addrs[lane] // 2:addrs[lane] // 2 + 8]
                row, col = kt * 32 + lane % 32, 16 * st + 8 * (lane // 32)
                assert (got == vals[row, col:col + 8]).all(), (kt, st, lane)
            assert conflict_cycles(addrs, 16, 4) == 0, (kt, st)


@pytest.mark.parametrize("d", [128, 64])
def test_v_operand_transposed_reads(dump, d):
    vals, lds = fill_tile(d, dump[d])
    tab = dump[d]
    for kt in range(BC // 32):
        for u in range(2):
            for dt in range(d // 32):
                got = np.zeros((64, 8), int)
                for sec in range(2):
                    addrs = [tab["v"][(dt, sec, lane)] + (32 * kt + 16 * u) * 2 * d
                             for lane in range(64)]
                    assert conflict_cycles(addrs, 32, 2) == 0, (kt, u, dt, sec)
                    for lane in range(64):
                        g, i = lane >> 4, lane & 15
                        for j in range(4):
                            src = 16 * g + 4 * j + (i >> 2)
                            got[lane, 4 * sec + j] = lds[addrs[src] // 2 + (i & 3)]
                # MFMA A operand of O^T = V^T P^T: lane l holds head-dim row
                # dt*32 + l % 32 and, in element e, the key the P^T operand
                # pairs with it: 16 u + 4 (l / 32) + (e & 3) + 8 (e >> 2)
                for lane in range(64):
                    for e in range(8):
                        key = 32 * kt + 16 * u + 4 * (lane >> 5) + (e & 3) + 8 * (e >> 2)
                        assert got[lane, e] == vals[key, dt * 32 + lane % 32], (kt, u, dt, lane)
