"""Launches whose tiles hold rows past the 20 register slabs in the 8 LDS
slabs, one per strip width 8 << lt columns: a group of R rows on such strips
(rps = 512 >> lt rows per slab) uses the LDS for 20 * rps < R <= 28 * rps.
Each case is (K, sizes, lt): the first size repeated makes enough tiles
that the launch keeps its widest strips (the library narrows them until
there is a tile per compute unit); the rest add ragged last slabs, empty
groups and short groups beside them. dim0_t cases have group sizes on the
16-row grid its outputs need."""

DIM0 = [
    (8200, [28] * 90 + [21, 27, 0, 5], 9),          # 4096-column strips, rps = 1
    (4104, [56] * 100 + [41, 55, 1], 8),            # 2048, rps = 2
    (2056, [96] * 86 + [81, 100, 0, 112, 7], 7),    # 1024, rps = 4
    (1032, [200] * 86 + [161, 224, 3], 6),          # 512, rps = 8
    (520, [400] * 86 + [321, 448, 16], 5),          # 256, rps = 16
    (264, [700] * 86 + [641, 896, 5, 0], 4),        # 128, rps = 32
]

# The transposed kernel picks strip widths by its 640 register rows, so only
# groups of 641 to 896 rows (and chunks of taller groups) on 128-column
# strips hold rows in LDS.
DIM0_T = [
    (264, [768] * 86 + [656, 896, 16, 0], 4),       # 128, rps = 32
    (520, [704] * 50 + [1792, 880, 16], 4),         # two-chunk teams of 896 rows beside them
]
