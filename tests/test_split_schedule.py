"""Model of the GEMM's persistent schedule with a split last round (CPU).

The kernel deals tiles to one workgroup per CU: XCD x = b mod 8 of workgroup b owns a
contiguous range of the tile order, its gx workgroups (jx = b / 8) take R = len / gx
full rounds, and with a work space the L = len mod gx tiles left for the last round
are split along K into s parts, part q of leftover tile j on workgroup jx = j + q L.
The owner (part s - 1) waits for the parts of workgroups x + 8 (j + q L), q < s - 1.
This test replays that integer arithmetic for many shapes and checks what the kernel
relies on:
* every (tile, k-step) is computed exactly once;
* parts are non-empty whole groups of the unrolled loop;
* each split tile's owner has the highest workgroup id of its parts (it waits only
  for workgroups that the in-order dispatcher started before it), and the ids it
  waits for are exactly its tile's other parts;
* partial slots (indexed by workgroup id) and flags are never shared within a call;
* the host's any_split() says "split" exactly when some tile is split.
"""
import pytest


def sched_of(b, G, tiles, nks, spg, split_max):
    X = min(G, 8)
    x, jx = b & 7, b >> 3
    gx = (G - x + 7) >> 3
    q, r = divmod(tiles, X)
    x0 = x * q + min(x, r)
    ln = q + (1 if x < r else 0)
    R, L = divmod(ln, gx)
    s = 1
    if split_max > 1 and L > 0:
        s = min(gx // L, split_max, nks // spg)
    nk_part = -(-(nks // spg) // s) * spg if s > 1 else nks
    if s > 1:
        s = -(-nks // nk_part)
    has_part = s > 1 and jx < L * s
    n_mine = R + (1 if has_part or (s == 1 and jx < L) else 0)
    units = []
    for i in range(n_mine):
        if has_part and i == R:
            j, qq = jx % L, jx // L
            k0 = qq * nk_part
            units.append(dict(tile=x0 + R * gx + j, k0=k0, k1=min(nks, k0 + nk_part), part=qq, s=s, j=j, L=L, x=x))
        else:
            units.append(dict(tile=x0 + jx + i * gx, k0=0, k1=nks, part=None))
    return units


def any_split(tiles, G, nks, spg):
    X = min(G, 8)
    for x in range(X):
        ln = tiles // X + (1 if x < tiles % X else 0)
        gx = (G - x + 7) // 8
        L = ln % gx
        if L > 0 and min(gx // L, 8, nks // spg) > 1:
            return True
    return False


CASES = [
    # tiles, G, nks, spg: the full-size workloads on 256 CUs, then small and odd ones
    (864, 256, 24, 2), (864, 256, 24, 4), (1536, 256, 24, 4), (1152, 256, 24, 4), (576, 256, 96, 2),
    (432, 256, 96, 2), (1056, 256, 64, 4), (768, 256, 32, 2), (2304, 256, 48, 4),
    (6, 256, 24, 4), (1, 256, 24, 4), (1, 256, 2, 2), (37, 256, 8, 2), (255, 256, 24, 4), (257, 256, 24, 4),
    (300, 304, 24, 4), (13, 80, 12, 2), (1000, 256, 6, 2), (3, 5, 24, 4), (40, 256, 4, 4),
]


@pytest.mark.parametrize("tiles,G,nks,spg", CASES, ids=[f"t{c[0]}-G{c[1]}-k{c[2]}-g{c[3]}" for c in CASES])
def test_every_tile_and_k_step_once(tiles, G, nks, spg):
    cover = {}
    parts = {}      # tile -> {part q: workgroup}
    for b in range(G):
        for u in sched_of(b, G, tiles, nks, spg, 8):
            assert 0 <= u["tile"] < tiles
            assert u["k1"] > u["k0"] and u["k0"] % spg == 0 and (u["k1"] - u["k0"]) % spg == 0
            for k in range(u["k0"], u["k1"]):
                key = (u["tile"], k)
                assert key not in cover, f"{key} computed twice"
                cover[key] = b
            if u["part"] is not None:
                parts.setdefault(u["tile"], {})[u["part"]] = (b, u)
    assert len(cover) == tiles * nks
    split_tiles = 0
    for t, ps in parts.items():
        s = next(iter(ps.values()))[1]["s"]
        assert sorted(ps) == list(range(s)), (t, sorted(ps))
        owner_b, owner = ps[s - 1]
        assert owner_b == max(b for b, _ in ps.values()), "the owner has the highest workgroup id"
        waits = [owner["x"] + 8 * (owner["j"] + q * owner["L"]) for q in range(s - 1)]
        assert waits == [ps[q][0] for q in range(s - 1)], "the owner waits for exactly its tile's parts"
        split_tiles += 1
    assert any_split(tiles, G, nks, spg) == (split_tiles > 0)


def test_full_rounds_unchanged_without_a_work_space():
    # split_max = 1: the plain schedule, every unit a whole tile
    for tiles, G, nks, spg in CASES:
        seen = set()
        for b in range(G):
            for u in sched_of(b, G, tiles, nks, spg, 1):
                assert u["part"] is None and (u["k0"], u["k1"]) == (0, nks)
                assert u["tile"] not in seen
                seen.add(u["tile"])
        assert len(seen) == tiles


def test_split_shapes_of_the_workloads():
    """The last round of the DiT shapes that leave one partly empty (per XCD on 256 CUs)."""
    def split_factor(tiles, nks, spg):
        s_max = 1
        for b in range(256):
            for u in sched_of(b, 256, tiles, nks, spg, 8):
                if u["part"] is not None:
                    s_max = max(s_max, u["s"])
        return s_max
    assert split_factor(864, 24, 2) == 2       # QK-RMSNorm hd128, 4608 x 9216 x 3072, 256 x 192 tiles
    assert split_factor(1152, 24, 4) == 2      # GELU-tanh 4608 x 12288 x 3072, 4 x 1 grid
    assert split_factor(576, 96, 2) == 4       # gated residual 9216 x 3072 x 12288, 256 x 192 tiles
    assert split_factor(1536, 24, 4) == 1      # the headline: exactly 6 rounds, nothing to split
