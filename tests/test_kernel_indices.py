"""CPU replay of the global-memory index arithmetic of the grouped-family
kernels (the MLP kernel of atlas_mem_grouped.hip, the linear kernels of
atlas_mem_linear.hip and the phi / Q1 kernels of atlas_mem_phi.h), of the
prologue's GEMM kernels and of the streamed kernel's state blocks: every
offset a lane forms is recomputed here, for every wave, lane, chunk and tile
the kernels visit, at the library's shapes and ragged lengths, and checked
against the size of the array it addresses.  Accesses through range-checked
buffer descriptors are checked too, so that an index out of range (which the
hardware would silently turn into a zero) is caught as a bug.

The formulas restate the kernels' own expressions; a change of a kernel's
indexing must be mirrored here (the test then proves the new indices before
any GPU run).
"""
import numpy as np
import pytest

BC = 64
PHI_IDENTITY, PHI_POLY2, PHI_RAW_POLY2 = 0, 1, 2


def feature_dim(phi, dk, pd):
    if phi == PHI_IDENTITY:
        return dk
    if phi == PHI_POLY2:
        return dk + dk * (dk + 1) // 2
    return dk + pd + pd * (pd + 1) // 2


def align(x, a=256):
    return (x + a - 1) // a * a


LANE = np.arange(64)
G4, C16 = LANE >> 4, LANE & 15


def check(offs, size, what):
    offs = np.asarray(offs)
    if offs.size:
        assert offs.min() >= 0 and offs.max() < size, (what, int(offs.min()), int(offs.max()), size)


# ----------------------------------------------------------------------------- MLP kernel
def grouped_mlp(phi, dk, pd, dv, h, g, n, c):
    D = feature_dim(phi, dk, pd)
    DP = (D + 63) // 64 * 64
    WP, HL = 128, h // g
    NFW, NDW, RW, RQ = DP // 64, dv // 64, WP // g, BC // g
    nch = -(-n // BC)
    NR = nch * BC + BC
    W = BC + c - 1
    assert HL == 16 and W <= WP
    xr_size = NR * DP * 2          # bytes: key rows, the feature-major copy
    xq_size = nch * BC * DP * 2
    xy_size = 2 * g * WP * dv * 4
    xo_size = 2 * g * BC * dv * 4
    state_w = (h * D + dv * h) * 4
    npair = RW * (dv // 4)
    nsplit = 256 // npair
    per = g // nsplit
    npair_o = RQ * (dv // 4)
    nsplit_o = 256 // npair_o
    per_o = g // nsplit_o
    for pm in range(g):
        j0 = HL * pm
        for wave in range(4):
            fb = 16 * NFW * wave
            # state slices (kZeroOffset for padded features is out of range on purpose)
            for t in range(NFW):
                f = fb + 16 * t + C16
                for r in range(4):
                    off = ((j0 + 4 * G4 + r) * D + f) * 4
                    check(off[f < D], state_w, "W1 state")
            for t in range(NDW):
                for r in range(4):
                    check((h * D + (16 * (NDW * wave + t) + 4 * G4 + r) * h + j0 + C16) * 4, state_w, "W2 state")
            R0, Q0 = 32 * wave, 16 * wave
            for ch in range(nch):
                t0 = ch * BC
                sl = ch & 1
                for ks in range(DP // 32):
                    for mt in range(2):
                        check(((t0 + R0 + 16 * mt + C16) * DP + 32 * ks + 8 * G4) * 2 + 15, xr_size, "forward X")
                    check(((t0 + Q0 + C16) * DP + 32 * ks + 8 * G4) * 2 + 15, xq_size, "query rows")
                yb = ((sl * g + pm) * WP) * dv * 4
                for mt in range(2):
                    for nt in range(dv // 16):
                        check(yb + ((R0 + 16 * mt + C16) * dv + 16 * nt + 4 * G4) * 4 + 15, xy_size, "Y partials")
                yo = ((sl * g + pm) * BC) * dv * 4
                for nt in range(dv // 16):
                    check(yo + ((Q0 + C16) * dv + 16 * nt + 4 * G4) * 4 + 15, xo_size, "output partials")
                for t in range(NFW):
                    f = fb + 16 * t + C16
                    for s in range(WP // 32):
                        check((f * NR + t0 + 32 * s + 8 * G4) * 2 + 15, xr_size, "update X^T")
        # reduce-scatter and output reduction (all 256 threads)
        tid = np.arange(256)
        e, hh = tid % npair, tid // npair
        w = pm * RW + e // (dv // 4)
        o4 = (e % (dv // 4)) * 4
        assert w.max() < WP
        for sl in range(2):
            for u in range(per):
                check((sl * g * WP * dv + w * dv + o4 + (hh * per + u) * WP * dv) * 4 + 15, xy_size, "reduce-scatter")
            check(((sl * WP + w) * dv + o4) * 2 + 7, 2 * WP * dv * 2, "D2 rows")
        e, hh = tid % npair_o, tid // npair_o
        qq = pm * RQ + e // (dv // 4)
        o4 = (e % (dv // 4)) * 4
        assert qq.max() < BC
        for pc in range(2):
            for u in range(per_o):
                check(((pc & 1) * g * BC * dv + qq * dv + o4 + (hh * per_o + u) * BC * dv) * 4 + 15, xo_size,
                      "output reduction")
        for ch in range(nch):
            t0, te = ch * BC, min(n, ch * BC + BC) - 1
            rows = t0 + qq
            check(((rows[rows <= te]) * dv + o4[rows <= te]) * 2 + 7, n * dv * 2, "output rows")
            # window values of the reduce-scatter rows
            e = tid % npair
            w = pm * RW + e // (dv // 4)
            i = t0 - (c - 1) + w
            ok = (w < W) & (i <= te)
            check((i[ok & (i >= 0)] * dv) * 2, n * dv * 2, "value rows")
            hi = (c - 1 + i[ok & (i < 0) & (i >= -(c - 1))])
            if hi.size:
                check(hi * dv * 4, (c - 1) * dv * 4, "halo values")


GROUPED_SHAPES = {"atlas_long": (PHI_RAW_POLY2, 128, 32, 128, 512, 32), "layer_scale": (PHI_IDENTITY, 128, 0, 128, 512, 32),
                  "mlp64": (PHI_IDENTITY, 64, 0, 64, 256, 16)}


@pytest.mark.parametrize("name", list(GROUPED_SHAPES))
@pytest.mark.parametrize("n,c", [(1, 1), (37, 64), (64, 32), (65, 64), (209, 33), (4 * 64, 64)])
def test_grouped_mlp_indices(name, n, c):
    grouped_mlp(*GROUPED_SHAPES[name], n, c)


# ----------------------------------------------------------------------------- linear kernels
def img_pos(o, f, nout):
    return ((f >> 2) * 16 + (o & 15)) * (4 * nout) + (o >> 4) * 4 + (f & 3)


def linear(phi, dk, pd, dv, wp, n, c):
    D = feature_dim(phi, dk, pd)
    DP = (D + 63) // 64 * 64
    NOT, NFT, NWT = dv // 16, DP // 16, wp // 16
    YPW, FPW = NOT * NWT // 4, NFT // 4
    assert BC + c - 1 <= wp
    nch = -(-n // BC)
    NR = nch * BC + BC
    img_elems = nch * 2 * dv * DP
    dg_elems = nch * wp * dv
    xr_size = NR * DP * 2
    # X^T staging: J 1-KB instructions cover R rows of wp*2 bytes
    rb = wp * 2
    J = rb // np.gcd(rb, 1024)
    R = J * 1024 // rb
    NSB = DP // R
    assert DP % R == 0 and NSB % 4 == 0
    # the image order is a bijection onto [0, dv * DP)
    o, f = np.meshgrid(np.arange(dv), np.arange(DP), indexing="ij")
    pos = img_pos(o, f, NOT)
    assert np.array_equal(np.sort(pos.ravel()), np.arange(dv * DP))
    for wave in range(4):
        for m in range(FPW):
            f0 = 16 * (wave + 4 * m) + 4 * G4
            q0 = img_pos(C16, f0, NOT)
            assert (q0 % 8 == 0).all()
            for chn in range(nch):
                check(chn * 2 * dv * DP + dv * DP + q0 + 8 * (NOT // 2 - 1) + 7, img_elems, "S image")
        for ch in range(nch):
            t0 = ch * BC
            for u in range(YPW):
                ot, wt = (wave + 4 * u) % NOT, (wave + 4 * u) // NOT
                w = 16 * wt + C16
                check(((ch * wp + w) * dv + 16 * ot + 4 * G4) + 3, dg_elems, "D rows")
                for s in range(DP // 32):
                    check(((t0 + 16 * wt + C16) * DP + 32 * s + 8 * G4) * 2 + 15, xr_size, "window X")
            for k in range(NSB // 4):
                sb = wave + 4 * k
                soff = (sb * R * NR + t0) * 2
                for j in range(J):
                    off = j * 1024 + LANE * 16
                    voff = (off // rb) * NR * 2 + off % rb
                    check(voff + soff + 15, xr_size, "X^T staging")
                    assert (sb * J + j) * 1024 + 1023 < DP * wp * 2
    # retrieval: the image operand as two 8-byte halves
    for ch in range(nch):
        for o_t in range(NOT):
            for s in range(DP // 32):
                q = img_pos(16 * o_t + C16, 32 * s + 8 * G4, NOT)
                check(dv * DP + q + 64 * NOT + 3, 2 * dv * DP, "retrieval image")


LINEAR_SHAPES = {"poly2_w96": (PHI_POLY2, 32, 32, 32, 96), "poly2_w128": (PHI_POLY2, 32, 32, 32, 128),
                 "id64_w64": (PHI_IDENTITY, 64, 0, 64, 64)}


@pytest.mark.parametrize("name", list(LINEAR_SHAPES))
@pytest.mark.parametrize("n", [1, 37, 64, 65, 209, 1024])
def test_linear_indices(name, n):
    shape = LINEAR_SHAPES[name]
    for c in (1, 16, 33, 64):
        if BC + c - 1 <= shape[-1]:
            linear(*shape, n, c)


# ----------------------------------------------------------------------------- phi and Q1 kernels
@pytest.mark.parametrize("phi,dk,pd,wp", [(PHI_RAW_POLY2, 128, 32, 128), (PHI_POLY2, 32, 32, 96), (PHI_IDENTITY, 64, 0, 64)])
@pytest.mark.parametrize("n", [1, 65, 209])
def test_phi_and_q1_indices(phi, dk, pd, wp, n):
    D = feature_dim(phi, dk, pd)
    DP = (D + 63) // 64 * 64
    nch = -(-n // BC)
    NR = nch * BC + BC
    assert NR % 32 == 0
    per_seq = NR // 32 + 2 * nch
    for blk in range(per_seq):
        keys = blk < NR // 32
        r0 = 32 * (blk if keys else blk - NR // 32)
        # the row pass: e = tid, tid + 256, ... < 32 DP / 8 -> row r0 + e / (DP / 8)
        e = np.arange(32 * (DP // 8))
        rows = r0 + e // (DP // 8)
        limit = NR if keys else nch * BC
        check((rows * DP + (e % (DP // 8)) * 8) * 2 + 15, limit * DP * 2, "phi rows")
        if keys:
            f = np.arange(DP)[:, None]
            t8 = np.arange(4)[None, :] * 8
            check(f * NR + r0 + t8 + 7, NR * DP, "feature-major keys")
    # Q1: query tile `wave`, all window tiles
    for ch in range(nch):
        t0 = ch * BC
        for wave in range(4):
            for s in range(DP // 32):
                check(((t0 + 16 * wave + C16) * DP + 32 * s + 8 * G4) * 2 + 15, nch * BC * DP * 2, "Q1 queries")
                for nt in range(wp // 16):
                    check(((t0 + 16 * nt + C16) * DP + 32 * s + 8 * G4) * 2 + 15, NR * DP * 2, "Q1 keys")


# ----------------------------------------------------------------------------- projection GEMM
def gemm_nt(M, N, K):
    """atlas_prologue_gemm.hip: tile order, LDS-direct load offsets with the
    granule swizzle, the zero-filled K tail and stages past the last, the
    fragment read offsets, and the output offsets."""
    BM = BN = 256
    BK, ROWB, GM = 64, 128, 4
    tiles_m, tiles_n = -(-M // BM), -(-N // BN)
    T = tiles_m * tiles_n
    T8 = -(-T // 8)
    seen = set()
    for blk in range(8 * T8):
        t = (blk & 7) * T8 + (blk >> 3)
        if t >= T:
            continue
        band = t // (GM * tiles_n)
        i = t - band * GM * tiles_n
        gm = min(GM, tiles_m - band * GM)
        tm, tn = band * GM + i % gm, i // gm
        assert 0 <= tm < tiles_m and 0 <= tn < tiles_n
        seen.add((tm, tn))
    assert len(seen) == T
    nk = -(-K // BK)
    ktail = K - (nk - 1) * BK
    far, zero_off = 0x40000000, 0x7FFFFF00
    g = [(LANE & 7) ^ (4 * p + (LANE >> 4)) for p in range(2)]
    voff = [(LANE >> 3) * K * 2 + (g[p] << 4) for p in range(2)]
    voff_last = [np.where(8 * g[p] < ktail, voff[p], zero_off) for p in range(2)]
    # the first tile of each operand (the largest valid row count; a partial
    # tile only shrinks its descriptor)
    size = {False: min(BM, M) * K * 2, True: min(BN, N) * K * 2}
    for wave in range(4):
        for s in range(nk + 2):
            kofs = s * ROWB if s < nk else far
            cover = set()
            for q in range(16):
                row = 64 * wave + 8 * (q & 7)
                vo = voff_last[q & 1] if s == nk - 1 else voff[q & 1]
                off = vo.astype(np.int64) + row * K * 2 + kofs
                assert off.max() < 2 ** 32
                dst = (s & 1) * 2 * BM * ROWB + (0 if q < 8 else BM * ROWB) + row * ROWB + LANE * 16
                assert dst.max() + 16 <= 4 * BM * ROWB
                inb = off < size[q >= 8]
                if s >= nk:
                    assert not inb.any()
                    continue
                r, k = off // (K * 2), (off % (K * 2)) // 2
                # an in-range granule lies inside its row, in this stage, below K
                assert (r[inb] == row + (LANE[inb] >> 3)).all()
                assert (k[inb] >= s * BK).all() and (k[inb] + 8 <= min(K, s * BK + BK)).all()
                # and lands in the swizzled slot of its granule
                rr = (dst % (BM * ROWB)) // ROWB
                slot = (dst % ROWB) // 16
                assert ((slot == (((k - s * BK) // 8) ^ ((rr >> 1) & 7))) | ~inb).all()
                cover.update((q >= 8, int(o)) for o in off[inb])
            if s < nk:
                # every granule of this wave's valid rows below K is loaded once
                want = min(BK, K - s * BK) // 8
                rows_a = max(0, min(64, M - 64 * wave))
                rows_b = max(0, min(64, N - 64 * wave))
                assert len(cover) == (rows_a + rows_b) * want
    for kk in range(2):
        fo = (LANE & 15) * ROWB + (((4 * kk + (LANE >> 4)) ^ ((LANE & 15) >> 1)) << 4)
        for r0 in range(0, 256, 16):
            r = r0 + (LANE & 15)
            assert (((fo % ROWB) // 16) == ((4 * kk + (LANE >> 4)) ^ ((r >> 1) & 7))).all()
            assert (r0 * ROWB + fo).max() + 16 <= BM * ROWB
    for wm in range(2):
        for wn in range(2):
            for i in range(8):
                col = 128 * wn + 16 * i + 4 * (LANE >> 4)
                for j in range(8):
                    row = 128 * wm + 16 * j + (LANE & 15)
                    vo = np.where(col < N, (row * N + col) * 2, zero_off)
                    assert vo.max() < 2 ** 31


@pytest.mark.parametrize("M,N,K", [(131072, 4672, 1536), (1000, 100, 64), (300, 260, 192), (64, 4, 8),
                                   (513, 1028, 1000), (256 * 9, 768, 1536 + 24)])
def test_projection_gemm_indices(M, N, K):
    gemm_nt(M, N, K)


def fused_prologue(B, N, dm, H, d, K, r):
    """The one-kernel prologue: row tiles along each sequence with a window of
    K - 1 recomputed rows, the P tile in LDS (16-byte granule swizzle), the
    epilogue's rows, heads, window reads, norm-part block and output offsets.
    Every output element is written exactly once."""
    BM = BN = 256
    halo = K - 1
    KP = 4 if K <= 4 else 8
    HD = H * d
    ncol = 3 * HD + 4 * r
    assert (3 * HD) % BN == 0
    tps = 1 + ((N - BM + (BM - halo) - 1) // (BM - halo) if N > BM else 0)
    tiles_n = -(-ncol // BN)
    DPL, HPT = d // 64, BN // d
    WPH = 4 // HPT
    TB = 16
    lds_p = 128 * 1024
    wave_floats = TB * 64 + TB
    lds_total = lds_p + 4 * wave_floats * 4
    assert lds_total <= 160 * 1024
    assert 4 * H * (r + 1) <= 4 * wave_floats   # the gate tile's V and b

    def ptile(t, c16):
        return t * 512 + ((c16 ^ (t & 15)) << 4)

    # the P tile writes: every (row, 8-byte quarter-granule) exactly once
    seen = set()
    for wave in range(4):
        wm, wn = wave >> 1, wave & 1
        for i in range(8):
            for j in range(8):
                t = 128 * wm + 16 * j + (LANE & 15)
                cg = 32 * wn + 4 * i + (LANE >> 4)
                a = np.array([ptile(int(tt_), int(c) >> 1) for tt_, c in zip(t, cg)]) + (cg & 1) * 8
                assert a.min() >= 0 and (a + 8).max() <= lds_p
                seen.update(int(x) for x in a)
    assert len(seen) == 256 * 64
    written = {m: np.zeros((B, H, N), np.int32) for m in range(3)}
    gates = np.zeros((4, B, H, N), np.int32)
    for b in range(B):
        for tt in range(tps):
            row0 = tt * (BM - halo)
            assert row0 < N and row0 * dm * 2 + 255 * dm * 2 + 0x40000000 < 2 ** 32
            nvalid = min(BM, N - row0)
            out_lo = 0 if tt == 0 else halo
            for tn in range(tiles_n):
                n0 = tn * BN
                if n0 >= 3 * HD:
                    for tid in range(256):
                        t = out_lo + tid
                        if t >= nvalid:
                            continue
                        for c in range(0, 4 * r, 4):
                            a = ptile(t, c >> 3) + (c & 4) * 2
                            assert a + 8 <= lds_p
                        for g in range(4):
                            gates[g, b, :, row0 + t] += 1
                    continue
                for wave in range(4):
                    hh, part = wave // WPH, wave % WPH
                    c0 = n0 + hh * d
                    m, h = c0 // HD, (c0 % HD) // d
                    assert m < 3 and h < H
                    ln = nvalid - out_lo
                    t_beg = out_lo + (part * ln) // WPH
                    t_end = out_lo + ((part + 1) * ln) // WPH
                    col = hh * d + LANE * DPL
                    assert ((col % 8) + DPL <= 8).all()
                    # window rows before the first: clamped at 0; rows the real
                    # taps reach lie in the tile (or precede the sequence)
                    assert t_beg - halo >= 0 or tt == 0
                    for t in list(range(max(0, t_beg - KP + 1), t_beg)) + list(range(t_beg, t_end)):
                        a = np.array([ptile(t, int(c) >> 3) for c in col]) + (col & 7) * 2
                        assert a.min() >= 0 and (a + 2 * DPL).max() <= lds_p
                    # the wave's norm parts and scales
                    base = lds_p + wave * wave_floats * 4
                    assert base + (TB * 64 + TB) * 4 <= lds_total
                    written[m][b, h, row0 + t_beg:row0 + t_end] += 1
                    chan = c0 + LANE * DPL
                    assert (chan + DPL - 1).max() < 3 * HD
    for m in range(3):
        assert (written[m] == 1).all(), m
    assert (gates == 1).all()


@pytest.mark.parametrize("B,N,dm,H,d,K,r", [(2, 37, 256, 2, 128, 4, 16), (1, 256, 512, 2, 128, 4, 16),
                                            (2, 257, 256, 2, 128, 4, 16), (1, 1000, 384, 2, 128, 4, 16),
                                            (2, 509, 256, 4, 64, 1, 4), (1, 777, 320, 4, 64, 8, 1),
                                            (1, 600, 512, 1, 256, 3, 8), (1, 16384, 1536, 12, 128, 4, 16)])
def test_fused_prologue_indices(B, N, dm, H, d, K, r):
    fused_prologue(B, N, dm, H, d, K, r)


# ----------------------------------------------------------------------------- streamed state blocks
# The streamed kernel (atlas_mem_stream.hip) keeps the state between passes in
# blocks, one per super tile J (HJ = 64 hidden units) and wave w: block
# J * 4 + w holds that wave's W1 rows [ND], S1 rows [ND], W2 values [NU][NDT],
# S2 values [NU][NDT] (fp32) and A, gelu'(Z) [NT] (bf16), each a 1 KB tile in
# lane order.  A tile access is lane offset 16 l, the tile's place within its
# 4 KB (immediate offset) and a wave-uniform scalar offset in 4 KB steps; the
# exchange slots follow the blocks.
STREAMED_SHAPES = [(128, 128, 512, 96), (128, 128, 512, 64), (128, 128, 384, 96), (128, 128, 256, 96),
                   (64, 64, 256, 64), (64, 64, 256, 96)]


@pytest.mark.parametrize("D,DV,H,WP", STREAMED_SHAPES)
def test_streamed_state_blocks(D, DV, H, WP):
    NW, HJ = 4, 64
    ND, NU, NDT, NT = D // 16, HJ // 16, DV // NW // 16, WP // 16
    TW1, TS1, TW2, TS2, TAG = 0, ND, 2 * ND, 2 * ND + NU * NDT, 2 * ND + 2 * NU * NDT
    NTB = TAG + NT
    SB = NTB * 1024
    ts_bytes = (H // HJ) * NW * SB
    # the fp32 state fills exactly the W1/S1/W2/S2 tiles of all blocks
    assert (H // HJ) * NW * (2 * ND + 2 * NU * NDT) * 1024 == 2 * H * D * 4 + 2 * DV * H * 4
    cover = np.zeros(ts_bytes // 16, dtype=np.int32)
    for J in range(H // HJ):
        for w in range(NW):
            tiles = ([TW1 + t for t in range(ND)] + [TS1 + t for t in range(ND)]
                     + [TW2 + a * NDT + b for a in range(NU) for b in range(NDT)]
                     + [TS2 + a * NDT + b for a in range(NU) for b in range(NDT)]
                     + [TAG + i for i in range(NT)])
            assert sorted(tiles) == list(range(NTB))
            for T in tiles:
                imm = (T % 4) * 1024
                assert imm < 4096   # the MUBUF immediate offset field
                offs = (J * NW + w) * SB + (T // 4) * 4096 + imm + 16 * LANE
                check(offs + 15, ts_bytes, ("block", J, w, T))
                cover[offs // 16] += 1
    # every 16 bytes of the blocks belong to exactly one lane of one tile
    assert (cover == 1).all()
