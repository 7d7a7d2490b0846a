"""Host-side check of the FP8 tile layout (fa_layout.hpp, head dim 128): the
direct-load fill of K and V tiles, the K operand reads of S^T = K Q^T and the
transposing V operand reads of O^T = V^T P^T, replayed on a model of the tile.
Checks that every lane receives the bytes its MFMA slots pair with the other
operand and that no read has an LDS bank conflict (64 banks of 4 bytes; 16
lanes per clock for 16-byte reads, 32 for 8-byte reads).  ds_read_b64_tr_b8 is
modelled as measured on the GPU: within each group of 16 lanes, result lane i
byte j is byte i % 8 of the 8 bytes addressed by source lane 2 j + (i / 8) % 2."""
import shutil
import subprocess

import numpy as np
import pytest

from test_lds_layout import INC, SRC, conflict_cycles

D, BC = 128, 64


@pytest.fixture(scope="module")
def tab(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("lds8") / "dump")
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", INC, SRC, "-o", exe], check=True)
    out = subprocess.run([exe, "fp8"], check=True, capture_output=True, text=True).stdout
    t = {"dma": {}, "k": {}, "v": {}, "p": {}}
    for line in out.splitlines():
        f = line.split()
        n = [int(x) for x in f[1:]]
        if f[0] == "dma":
            t["dma"][tuple(n[:3])] = tuple(n[3:])
        elif f[0] == "k":
            t["k"][tuple(n[:3])] = n[3]
        elif f[0] == "v":
            t["v"][tuple(n[:2])] = n[2]
        else:
            t["p"][tuple(n[:2])] = n[2]
    return t


def fill(tab, kind):
    vals = np.arange(BC * D).reshape(BC, D)
    lds = np.full(BC * D, -1)
    for inst in range(8):
        for lane in range(64):
            row, chunk = tab["dma"][(kind, inst, lane)]
            dst = inst * 1024 + lane * 16
            lds[dst:dst + 16] = vals[row, 16 * chunk:16 * chunk + 16]
    return vals, lds


@pytest.mark.parametrize("kind", [0, 1])
def test_fill_covers_every_byte_once(tab, kind):
    _, lds = fill(tab, kind)
    assert (lds >= 0).all() and len(np.unique(lds)) == lds.size


def test_p_slots_are_the_accumulator_keys(tab):
    for hh in range(2):
        keys = [tab["p"][(hh, s)] for s in range(32)]
        for s in range(32):
            kt, v = s >> 4, s & 15
            assert keys[s] == 32 * kt + (v & 3) + 8 * (v >> 2) + 4 * hh
    both = sorted(tab["p"][(hh, s)] for hh in range(2) for s in range(32))
    assert both == list(range(64))


def test_k_operand_reads(tab):
    vals, lds = fill(tab, 0)
    for kt in range(2):
        for st in range(2):
            for u in range(2):
                addrs = [tab["k"][(st, u, lane)] + kt * 32 * D for lane in range(64)]
                assert conflict_cycles(addrs, 16, 4) == 0, (kt, st, u)
                for lane in range(64):
                    got = lds[addrs[lane]:addrs[lane] + 16]
                    col = 64 * st + 32 * (lane >> 5) + 16 * u
                    assert (got == vals[32 * kt + lane % 32, col:col + 16]).all()


def test_v_operand_transposed_reads(tab):
    vals, lds = fill(tab, 1)
    for dt in range(4):
        got = np.zeros((64, 32), int)
        for q in range(4):
            addrs = [tab["v"][(dt, lane)] + 2048 * q for lane in range(64)]
            assert conflict_cycles(addrs, 32, 2) == 0, (dt, q)
            for lane in range(64):
                g, i = lane >> 4, lane & 15
                for j in range(8):
                    src = 16 * g + 2 * j + ((i >> 3) & 1)
                    got[lane, 8 * q + j] = lds[addrs[src] + (i & 7)]
        for lane in range(64):
            for s in range(32):
                key = tab["p"][(lane >> 5, s)]
                assert got[lane, s] == vals[key, 32 * dt + lane % 32], (dt, lane, s)
