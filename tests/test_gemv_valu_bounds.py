"""Host model of the one- and two-token decode kernel's memory accesses (CPU only).

nf4_gemv_valu_kernel (csrc/gemv.hip) computes every load address and every
partial-sum index per lane; a read past a buffer end is a GPU memory fault and
a missed or doubled partial is a wrong Y that only some shapes would show.
This model restates the kernel's work split (row workgroups: slice b % S, row
groups (b / S) * 8 + wave, 8 rows per wave, lane l on columns 32 l .. 32 l + 31
of a 2048-column slice; H workgroups: one per weight, slice and 16 ranks) and
its butterfly's writer lanes, and checks for grouped and ragged shapes that
  - every X, code, int8-scale, s2 and A read lies inside its buffer (the
    int8 codes as one aligned dword per lane when k % 256 == 0, and each
    lane's block inside the dword its shuffle reads),
  - every slice partial (slice, token, output column) and every H partial
    (weight, slice, token, rank) is written exactly once,
  - the partials fit in the workspace the forward sizes for the GEMV path.
It must be kept in step with the kernel's index arithmetic.
"""

import numpy as np
import pytest

VW, VCOL, VR = 8, 2048, 8     # waves per workgroup, columns per slice, rows per wave
GW, GB = 8, 16                # the MFMA kernel's constants that size the workspace


def _cdiv(a, b):
    return -(-a // b)


def _weight_of(gbase, nw, rg):
    i = 0
    for j in range(1, nw):
        if rg >= gbase[j]:
            i += 1
    return i


def _check(ds, k, M, rp):
    nw = len(ds)
    S = _cdiv(k, VCOL)
    ngi = [_cdiv(d, VR) for d in ds]
    gbase = np.concatenate([[0], np.cumsum(ngi)[:-1]]).astype(int)
    rbase = np.concatenate([[0], np.cumsum(ds)[:-1]]).astype(int)
    ngroups, dtot = sum(ngi), sum(ds)
    nbr = k // 64
    nrow_wg = _cdiv(ngroups, VW) * S
    nh_wg = nw * S * (rp // 16)
    lane = np.arange(64)
    tid = np.arange(64 * VW)
    part_hits = np.zeros(S * M * dtot, dtype=np.int64)
    hpart_hits = np.zeros((nw, S * M * rp), dtype=np.int64)
    MV = 1 if M == 1 else 2
    for b in range(nrow_wg + nh_wg):
        if b >= nrow_wg:    # H workgroup
            h = b - nrow_wg
            nrc = rp // 16
            cb, wsl = h % nrc, h // nrc
            wi, slice_ = wsl // S, wsl % S
            col0 = slice_ * VCOL + 32 * lane
            lok = col0 < k
            colc = np.where(lok, col0, 0)
            for m in range(MV):
                mr = m if m < M else 0
                x = mr * k + colc
                assert x.min() >= 0 and (x + 32).max() <= M * k, "H X read"
            for wave in range(VW):
                for tt in range(2):
                    t = 16 * cb + 2 * wave + tt
                    a = t * k + colc
                    assert (a + 32).max() <= rp * k, "A read"
                LGH = 5 if MV == 1 else 4
                idx = lane >> LGH
                tt, m = idx // MV, idx % MV
                wr = ((lane & ((1 << LGH) - 1)) == 0) & (m < M)
                for L in np.nonzero(wr)[0]:
                    hpart_hits[wi, (slice_ * M + m[L]) * rp + 16 * cb + 2 * wave + tt[L]] += 1
            continue
        slice_ = b % S
        xc = slice_ * VCOL + 8 * (tid & 255)
        for m in range(MV):
            mr = m if m < M else 0
            x = mr * k + np.where(xc < k, xc, 0)
            assert x.min() >= 0 and (x + 8).max() <= M * k, "X slice read"
        for wave in range(VW):
            rg = (b // S) * VW + wave
            rgc = min(rg, ngroups - 1)
            wi = _weight_of(gbase, nw, rgc)
            d = ds[wi]
            row0 = (rgc - gbase[wi]) * VR
            col0 = slice_ * VCOL + 32 * lane
            lok = col0 < k
            colc = np.where(lok, col0, 0)
            nb = d * k // 64
            if k % 256 == 0:   # aligned int8 codes: one dword per lane for the 8 rows
                rq = np.minimum(row0 + (lane >> 3), d - 1)
                off = np.minimum(slice_ * (VCOL // 64) + 4 * (lane & 7), nbr - 4)
                qa = rq * nbr + off
                assert qa.min() >= 0 and (qa + 4).max() <= nb and (qa % 4 == 0).all(), "int8 dword read"
                # each valid lane's block lies in the dword of lane 8 r + l / 8
                src_off = slice_ * (VCOL // 64) + 4 * (lane >> 3)
                blk_in_slice = slice_ * (VCOL // 64) + (lane >> 1)
                ok = lok
                assert (src_off[ok] <= blk_in_slice[ok]).all() and (blk_in_slice[ok] < src_off[ok] + 4).all()
                assert (src_off[ok] + 4 <= nbr).all(), "a valid lane's dword was clamped"
            for r in range(VR):
                row = min(row0 + r, d - 1)
                blk = row * nbr + (colc >> 6)
                assert blk.max() < nb and (blk >> 8).max() < _cdiv(nb, 256), "scale read"
                c = row * (k // 2) + (colc >> 1)
                assert (c + 16).max() <= d * k // 2, "code read"
            N = VR * MV
            LG = {8: 3, 16: 2}[N]
            idx = lane >> LG
            r, m = idx // MV, idx % MV
            wr = ((lane & ((1 << LG) - 1)) == 0) & (m < M) & (row0 + r < d) & (rg < ngroups)
            for L in np.nonzero(wr)[0]:
                part_hits[(slice_ * M + m[L]) * dtot + rbase[wi] + row0 + r[L]] += 1
    assert np.all(part_hits == 1), f"slice partials written {part_hits.min()}..{part_hits.max()} times"
    assert np.all(hpart_hits == 1), f"H partials written {hpart_hits.min()}..{hpart_hits.max()} times"
    s_old = _cdiv(k // 64, GB)
    ws_floats = s_old * M * dtot + nw * s_old * GW * M * rp
    assert S * M * dtot + nw * S * M * rp <= ws_floats, "workspace"


@pytest.mark.parametrize("ds,k,M,rp", [
    ([64], 64, 1, 16),               # one block per row
    ([104], 2112, 2, 16),            # a full slice + one block, 13 row groups
    ([8], 4096, 1, 16),              # padded ranks, one row group, two slices
    ([48], 11008, 2, 64),            # five full slices + 768 columns, four rank chunks
    ([16], 2048, 1, 128),            # r = 128, exactly one slice
    ([200], 960, 2, 16),             # one ragged slice
    ([11008], 4096, 1, 16),          # gate/up projection
    ([4096], 11008, 1, 16),          # down projection
    ([11008, 11008], 4096, 1, 16),   # gate and up in one call
    ([704, 704], 1088, 1, 16),       # grouped, ragged slice
    ([192, 320, 64], 2112, 2, 16),   # three sizes, two tokens
    ([8, 16, 24, 40], 6208, 2, 32),  # four weights, row groups smaller than a workgroup
])
def test_valu_gemv_accesses(ds, k, M, rp):
    _check(ds, k, M, rp)
