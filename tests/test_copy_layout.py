"""Host-side checks of the LDS tile addressing the attention kernels compile
(prism_internal.h: rm_swz, copy_offset, tr_offset, row_base, tr_base, tr_addr).  The header's
own functions are built into a host program (tests/layout_probe.cpp, hipcc host pass only)
and their outputs checked here against what the kernels rely on:

  * the direct global->LDS copies (lane l of copy i writes 16 bytes at 16 l of the copy's
    1 KB destination) place every source chunk where the swizzled layout rm_swz says the
    reads find it, and fill the [64][128] tile exactly once;
  * the transposed reads (ds_read_b64_tr_b16: in each 16-lane group lane i receives element
    i % 4 of the 8-byte pieces addressed by lanes 4j + i / 4, j = 0..3) give lane l, in
    register 4m + j, X[kb + 8m + 4 (l / 32) + j][db + l % 32], the MFMA operand order;
  * the hoisted XOR address forms equal the direct ones;
  * the row reads and the transposed reads of a half wave touch every LDS bank once.
"""
import os
import shutil
import subprocess
from collections import defaultdict

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("layout") / "probe")
    subprocess.run([hipcc, "-std=c++17", "--offload-host-only", "-x", "hip",
                    os.path.join(HERE, "layout_probe.cpp"), "-o", exe], check=True,
                   capture_output=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    rec = defaultdict(dict)
    for line in out.splitlines():
        kind, *vals = line.split()
        vals = [int(x) for x in vals]
        rec[kind][tuple(vals[:-1])] = vals[-1]
    return rec


def logical(off):
    """(row, column) of the 16-bit element stored at byte offset off of a swizzled tile."""
    row, pos = off // 256, (off % 256) // 16
    swz = ((row & 3) << 2) | ((row >> 2) & 3)
    return row, 8 * (pos ^ swz) + (off % 16) // 2


def test_copies_land_where_the_reads_look(probe):
    rm = probe["rm"]
    seen = set()
    for (r0, lane), c0 in probe["copy"].items():
        for i in range(4):
            src = (c0 ^ (16 * i)) + 1024 * i        # the lane's source offset in copy i
            dst = (r0 // 16) * 4096 + 1024 * i + 16 * lane
            assert src % 16 == 0 and 0 <= src < 16384
            # the 16 source bytes are row src // 256, chunk (src % 256) // 16 of the unit
            assert dst == rm[(src // 256, (src % 256) // 16)], (r0, lane, i)
            assert dst not in seen
            seen.add(dst)
    assert seen == set(range(0, 16384, 16))


def test_transposed_reads_give_the_operand_order(probe):
    tr = probe["tr"]
    for kb in range(0, 64, 16):
        for db in range(0, 128, 32):
            for m in range(2):
                pieces = [logical(tr[(kb, db, lane, m)]) for lane in range(64)]
                for lane in range(64):
                    g0 = lane & ~15
                    i = lane & 15
                    for j in range(4):
                        row, col = pieces[g0 + 4 * j + i // 4]
                        got = (row, col + i % 4)
                        want = (kb + 8 * m + 4 * (lane // 32) + j, db + lane % 32)
                        assert got == want, (kb, db, m, lane, j)


def test_hoisted_addresses_equal_direct_ones(probe):
    assert probe["xor_row"][()] == 0
    assert probe["xor_tr"][()] == 0


def test_half_wave_reads_are_free_of_bank_conflicts(probe):
    rm, tr = probe["rm"], probe["tr"]
    # row reads: 16 lanes read chunk c of 16 consecutive rows (16 bytes = 4 banks each)
    for r0 in range(0, 64, 16):
        for c in range(16):
            banks = [(rm[(r0 + k, c)] // 4 + b) % 64 for k in range(16) for b in range(4)]
            assert len(set(banks)) == 64, (r0, c)
    # transposed reads: 32 lanes read 8 bytes (2 banks) each
    for (kb, db, lane, m), off in tr.items():
        if lane % 32:
            continue
        banks = [(tr[(kb, db, lane + k, m)] // 4 + b) % 64 for k in range(32) for b in range(2)]
        assert len(set(banks)) == 64, (kb, db, lane, m)
