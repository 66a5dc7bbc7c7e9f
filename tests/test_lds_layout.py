"""LDS tile permutations (csrc/tiles.h) against a 64-bank model, on the host.

The permutations are restated here from their definition (chunk c of row r
at slot c ^ swz(r)) and each access pattern the kernels issue is replayed
on a model of 64 four-byte banks: a 16-byte read serves 16 lanes per
cycle, an 8-byte read 32; an access is conflict-free when no bank is asked
for two different words in one cycle.  The transposing read's lane
addressing is the one the kernels use (lane t of a 16-lane group addresses
row key0 + t/4, columns 32 dt + 16 (group % 2) + 4 (t % 4)).
"""

import pytest


def swz(D, kind, r):
    if D == 128:
        return {"k": r & 15, "v": (r & 3) << 2, "kv": ((r & 3) << 2) | ((r >> 2) & 3)}[kind]
    return {"k": (r >> 1) & 7, "v": ((r >> 1) & 1) << 2, "kv": (((r >> 1) & 1) << 2) | ((r >> 2) & 3)}[kind]


def worst_degree(addrs, width):
    lanes_per_cycle = 256 // width
    worst = 1
    for s in range(0, 64, lanes_per_cycle):
        banks = {}
        for a in addrs[s:s + lanes_per_cycle]:
            for k in range(width // 4):
                dw = a // 4 + k
                banks.setdefault(dw % 64, set()).add(dw)
        worst = max(worst, max(len(v) for v in banks.values()))
    return worst


def row_reads(D, kind):
    """16-byte operand reads: lane (j, h) reads row j (+32 t), chunk 2 s + h."""
    rb = 2 * D
    return [[(32 * t + l % 32) * rb + 16 * ((2 * s + l // 32) ^ swz(D, kind, 32 * t + l % 32)) for l in range(64)]
            for t in range(2) for s in range(D // 16)]


def tr_reads(D, kind):
    rb = 2 * D
    out = []
    for s in range(4):
        for hi in (0, 8):
            for dt in range(D // 32):
                addrs = []
                for l in range(64):
                    g, tg, h = l // 16, l % 16, l // 32
                    row = 16 * s + 4 * h + tg // 4 + hi
                    col = 32 * dt + 16 * (g % 2) + 4 * (tg % 4)
                    c, half = col // 8, (col // 4) % 2
                    addrs.append(row * rb + 16 * (c ^ swz(D, kind, row)) + 8 * half)
                out.append(addrs)
    return out


@pytest.mark.parametrize("D", [64, 128])
def test_permutations_are_bijections_on_chunks(D):
    ch = D // 8
    for kind in ("k", "v", "kv"):
        for r in range(64):
            assert sorted(c ^ swz(D, kind, r) for c in range(ch)) == list(range(ch))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["k", "kv"])
def test_row_reads_conflict_free(D, kind):
    assert max(worst_degree(a, 16) for a in row_reads(D, kind)) == 1


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["v", "kv"])
def test_transposing_reads_conflict_free(D, kind):
    assert max(worst_degree(a, 8) for a in tr_reads(D, kind)) == 1


def test_unpermuted_tile_would_conflict():
    # the model is not vacuous: without the permutation the same reads collide
    D = 128
    plain = [[(32 * t + l % 32) * 2 * D + 16 * (2 * s + l // 32) for l in range(64)] for t in range(2) for s in range(8)]
    assert max(worst_degree(a, 16) for a in plain) > 1


# The XOR-split offsets the backward kernels use in place of the
# definitions above (restated from csrc/tiles.h col8_parts and the row-read
# form base + ((32 s) ^ lane bits)); they must give the same byte addresses.

def col8_parts(D, kind, l):
    tg, h = l % 16, l // 32
    c0, half = 2 * ((l // 16) % 2) + ((tg >> 1) & 1), tg & 1
    r1 = 4 * h + tg // 4
    r2 = r1 + 8
    p1, p2 = swz(D, kind, r1), swz(D, kind, r2)
    return (2 * r1 * D + 16 * (c0 ^ (p1 & 3)) + 8 * half, 16 * (p1 & 12),
            2 * r2 * D + 16 * (c0 ^ (p2 & 3)) + 8 * half, 16 * (p2 & 12))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["k", "v", "kv"])
def test_xor_split_transposing_offsets(D, kind):
    rb = 2 * D
    for l in range(64):
        A1, B1, A2, B2 = col8_parts(D, kind, l)
        g, tg, h = l // 16, l % 16, l // 32
        for s in range(4):
            for dt in range(D // 32):
                col = 32 * dt + 16 * (g % 2) + 4 * (tg % 4)
                c, half = col // 8, (col // 4) % 2
                for hi, (A, B) in ((0, (A1, B1)), (8, (A2, B2))):
                    row = 16 * s + 4 * h + tg // 4 + hi
                    want = row * rb + 16 * (c ^ swz(D, kind, row)) + 8 * half
                    assert A + ((64 * dt) ^ B) + 32 * D * s == want


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["k", "kv"])
def test_xor_split_row_offsets(D, kind):
    rb = 2 * D
    for l in range(64):
        j, h = l % 32, l // 32
        for t in range(2):
            row = 32 * t + j
            y = 16 * (h ^ swz(D, kind, j))  # rows j and 32 + j share the permutation
            for s in range(D // 16):
                want = row * rb + 16 * ((2 * s + h) ^ swz(D, kind, row))
                assert j * rb + 64 * D * t + ((32 * s) ^ y) == want
