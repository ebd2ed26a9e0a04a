"""Host-side checks of the index arithmetic the attention kernels' global->LDS copies rely
on (prism_internal.h, copy_offset / copy_rows16): a [64][128] 16-bit tile is stored with
16-byte chunk c of row r at chunk c ^ swz(r), swz(r) = 4 (r % 4) + (r / 4) % 4; lane l of copy
i of a wave whose share starts at row r0 (a multiple of 16) fetches chunk (l % 16) ^ swz(r)
of row r = r0 + 4 i + l / 16 and writes it at 16 l of the copy's 1 KB destination."""
import itertools


def swz(r):
    return ((r & 3) << 2) | ((r >> 2) & 3)


def lane_offset(r0, i, lane):
    r = r0 + 4 * i + (lane >> 4)
    return r * 256 + (((lane & 15) ^ swz(r)) << 4)


def test_offsets_follow_from_the_first_copy():
    # copy i of a lane reads at (c0 ^ 16 i) + 1024 i, c0 being copy 0's offset
    for r0, lane, i in itertools.product(range(0, 64, 16), range(64), range(4)):
        c0 = lane_offset(r0, 0, lane)
        assert (c0 ^ (16 * i)) + 1024 * i == lane_offset(r0, i, lane), (r0, lane, i)


def test_copies_fill_the_swizzled_tile_exactly_once():
    # the 4 waves x 4 copies x 64 lanes land every stored chunk of the tile once, and the
    # chunk stored at LDS position p of row r is the source chunk whose swizzled position is p
    seen = {}
    for r0, i, lane in itertools.product(range(0, 64, 16), range(4), range(64)):
        src = lane_offset(r0, i, lane)
        dst = (r0 // 16) * 4096 + 1024 * i + 16 * lane   # LDS byte offset in the tile
        assert dst not in seen
        seen[dst] = src
    assert sorted(seen) == list(range(0, 16384, 16))
    for dst, src in seen.items():
        r, pos = dst // 256, (dst % 256) // 16
        sr, sc = src // 256, (src % 256) // 16
        assert sr == r and sc ^ swz(r) == pos
