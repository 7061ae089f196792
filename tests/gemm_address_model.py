"""Host model of the bf16 grouped GEMM's addressing (csrc/gemm_fast.h), for
the bounds test: the tile decode of every workgroup, the byte offsets of
every direct-to-LDS copy over every k-step, the output stores and the y
exponent index, mirrored from the kernel and checked against the buffers
they address.  Test infrastructure: it checks the kernel's index arithmetic,
not its results (the GPU parity tests do that)."""
from __future__ import annotations

import numpy as np

XCDS, Y_BLOCK = 8, 256


class Cfg:
    """Cfg<MODE, BM, BN, BK, STAGES=2, WM=4, WN=2, SB=2> of gemm_fast.h."""

    def __init__(self, mode, BM, BN, BK, WM=4, WN=2):
        self.mode, self.BM, self.BN, self.BK, self.WM, self.WN = mode, BM, BN, BK, WM, WN
        self.NW = WM * WN
        self.CPR = BK // 8
        self.RPI = 64 // self.CPR
        assert BM % (self.RPI * self.NW) == 0 and BN % (self.RPI * self.NW) == 0
        self.A_PER_WAVE, self.B_PER_WAVE = BM // self.RPI // self.NW, BN // self.RPI // self.NW
        self.HCOLS = BN // 2 if mode == "w13" else BN
        assert (2 * BM + 2 * BN) * BK * 2 <= 160 * 1024


# the instantiations of gemm.hip and the rule that picks them
W13, W13_NARROW = Cfg("w13", 320, 256, 64), Cfg("w13", 320, 64, 64)
DOWN, DOWN_K32 = Cfg("down", 320, 256, 64), Cfg("down", 256, 256, 32)


def configs(Im, Is=0):
    w13 = W13 if Im % 128 == 0 and Is % 128 == 0 else W13_NARROW
    down = DOWN if Im % 64 == 0 and Is % 64 == 0 else DOWN_K32
    return w13, down


def swz(cpr, row):
    return (row // (16 // cpr)) % cpr


def tiles(C, offsets, E, n_tiles, x_rows, x_ntiles):
    """decode_wave (equal-height m-tiles, XCD-contiguous logical ranges) for
    every workgroup of the launch grid."""
    cnt = np.diff(offsets)
    mt = (cnt + C.BM - 1) // C.BM
    t = mt * n_tiles
    incl = np.cumsum(t)
    total = int(incl[-1]) if E else 0
    x_mt = (x_rows + C.BM - 1) // C.BM
    allt = total + x_mt * x_ntiles
    R = int(offsets[-1])
    max_mt = max(1, (R + E * (C.BM - 1)) // C.BM)
    ntl = max_mt * n_tiles + x_mt * x_ntiles
    grid = (ntl + XCDS - 1) // XCDS * XCDS
    per = (allt + XCDS - 1) // XCDS
    out = []
    for b in range(grid):
        xcd, slot = b % XCDS, b // XCDS
        L = xcd * per + slot
        if not (slot < per and L < allt):
            continue
        xt = L >= total
        if xt:
            local, s_mt, s_off, s_cnt, e = L - total, x_mt, 0, x_rows, E
        else:
            e = int(np.argmax(incl > L))
            local, s_mt, s_off, s_cnt = L - (incl[e] - t[e]), mt[e], offsets[e], cnt[e]
        mts = max(int(s_mt), 1)
        rows = (((s_cnt + mts - 1) // mts + 15) & ~15)
        m0 = int(s_off + (local % mts) * rows)
        out.append(dict(e=int(e), xt=bool(xt), m0=m0, seg_end=int(min(m0 + rows, s_off + s_cnt)), nt=int(local // mts)))
    return out


def check(C, T, H, E, k, Im, mu, perm, offsets, Is=0):
    """Every address of one launch of configuration C in bounds, every output
    chunk written.  perm / offsets: a valid routing of the layer."""
    R = T * k
    n_tiles = mu * (Im // C.HCOLS) if C.mode == "w13" else (H + C.BN - 1) // C.BN
    x_ntiles = 0 if not Is else (Is // C.HCOLS if C.mode == "w13" else (H + C.BN - 1) // C.BN)
    lanes = np.arange(64)
    waves = np.arange(C.NW)[:, None]
    lrow, lpos = lanes // C.CPR, lanes % C.CPR
    covered = {False: [], True: []}
    for ti in tiles(C, offsets, E, n_tiles, T if Is else 0, x_ntiles):
        xt = ti["xt"]
        Im_, mu_ = (Is, 1) if xt else (Im, mu)
        lda = H if C.mode == "w13" else mu_ * Im_
        assert lda % C.BK == 0
        KT = lda // C.BK
        if C.mode == "w13":
            per_micro = Im_ // C.HCOLS
            micro, n0 = ti["nt"] // per_micro, (ti["nt"] % per_micro) * C.HCOLS
            a_size, b_size = T * H, (2 * Is * H if xt else mu * E * 2 * Im * H)
        else:
            micro, n0 = 0, ti["nt"] * C.BN
            a_size, b_size = (T * Is if xt else R * mu * Im), (H * Is if xt else mu * E * H * Im)
        eb = 0 if xt else ti["e"]
        a_rows = min(C.BM, (ti["seg_end"] - ti["m0"] + 15) & ~15)
        # A copies
        for i in range(C.A_PER_WAVE):
            g = waves + C.NW * i
            row = g * C.RPI + lrow
            live = np.broadcast_to(g * C.RPI < a_rows, row.shape)
            c = lpos ^ swz(C.CPR, row)
            p = np.minimum(ti["m0"] + row, ti["seg_end"] - 1)
            if C.mode == "w13":
                r = (p if xt else perm[p] // k) * H
            else:
                r = p * lda
            off = r + c * 8
            if not live.any():
                continue  # this load's row groups lie past the tile's rows: skipped
            assert (off[live] * 2 < 2 ** 32).all()
            for kt in (0, KT - 1):
                lo = kt * C.BK + off[live]
                assert lo.min() >= 0 and (lo + 8).max() <= a_size
                assert ((lo >= r[live]) & (lo + 8 <= r[live] + lda)).all()
        # B copies
        for i in range(C.B_PER_WAVE):
            row = (waves + C.NW * i) * C.RPI + lrow
            c = lpos ^ swz(C.CPR, row)
            if C.mode == "w13":
                half = C.BN // 2
                wrow = np.where(row < half, n0 + row, Im_ + n0 + (row - half))
                base0 = (micro * E + eb) * 2 * Im_ * H
                off = wrow * H + c * 8
                for kt in (0, KT - 1):  # linear in kt
                    lo = base0 + kt * C.BK + off
                    assert lo.min() >= base0 and (lo + 8).max() <= base0 + 2 * Im_ * H <= b_size
            else:
                wrow = np.minimum(row, H - 1 - n0)
                off = wrow * Im_ + c * 8
                for kt in range(KT):
                    kg = kt * C.BK
                    assert kg % Im_ + C.BK <= Im_, "a k-step crosses a micro-shard boundary"
                # linear in kt within a micro-shard: its first and last k-steps
                per = Im_ // C.BK
                for kt in sorted({q * per for q in range(mu_)} | {q * per + per - 1 for q in range(mu_)}):
                    kg = kt * C.BK
                    mm = kg // Im_
                    blk = (mm * E + eb) * H * Im_
                    lo = blk + n0 * Im_ + (kg - mm * Im_) + off
                    assert lo.min() >= blk and (lo + 8).max() <= blk + H * Im_ <= b_size
        # output stores (whole 16-byte pieces) and y exponents
        OC = C.HCOLS
        ldc = mu_ * Im_ if C.mode == "w13" else H
        col0 = micro * Im_ + n0 if C.mode == "w13" else n0
        cols = col0 + np.arange(0, OC, 8)
        if C.mode == "down":
            cols = cols[cols < ldc]
        assert (cols + 8 <= ldc).all()
        prow = np.arange(ti["m0"], ti["seg_end"])
        assert prow.size == 0 or prow.max() < (T if xt else R)
        covered[xt].append((prow[:, None] * ldc + cols[None, :]).ravel())
        if C.mode == "down" and prow.size:
            nb = (ldc + Y_BLOCK - 1) // Y_BLOCK
            assert (prow.max() * nb + col0 // Y_BLOCK) < (T if xt else R) * nb
    # every 16-byte piece of the output written exactly once
    for xt, rows in ((False, R), (True, T if Is else 0)):
        if rows == 0:
            continue
        ldc = (mu * Im if not xt else Is) if C.mode == "w13" else H
        want = np.arange(rows)[:, None] * ldc + np.arange(0, ldc, 8)[None, :]
        got = np.sort(np.concatenate(covered[xt]) if covered[xt] else np.zeros(0, np.int64))
        assert got.size == want.size and np.array_equal(got, np.sort(want.ravel())), "output pieces"
