"""Host model of the fused GEMM's fetch addresses (CPU only).

The fused dequant-GEMM fetches its In tiles, packed codes and scale words by
LDS DMA from addresses it computes per lane; a fetch past a buffer end is a
GPU memory fault, not a wrong number. This model restates, for every lane of
the eight waves (each fetches an eighth of the In tile; waves 0-3 fetch the
codes, waves 4-7 the scale words), tile and step the kernel issues (the prologue fetches steps 0-1 of In and
0-2 of codes unconditionally, clamping addresses), the address arithmetic of
csrc/gemm.hip and checks that each fetch lies inside its buffer, for the
workload shapes, the ragged test shapes and one-step contractions (the case
where the prologue's clamp steps back from past the end). It must be kept in
step with the kernel's fetch plan.
"""

import numpy as np
import pytest

BN, BM, BK = 128, 256, 64


def _cdiv(a, b):
    return -(-a // b)


def _fetches_in_bounds(d, k, M, mode, dq):
    Ntot, Ktot = (d, k) if mode == 0 else (k, d)
    nk = _cdiv(Ktot, BK)
    tid = np.arange(512)
    lane, wave = tid & 63, tid >> 6
    cw, sw = wave < 4, wave >= 4            # code and scale fetching waves
    p = 64 * (wave & 3) + lane              # code DMA lane
    e = 64 * (wave & 1) + lane              # scale DMA entry
    nb, ng = d * k // 64, _cdiv(d * k // 64, 256)
    x_steps = sorted({0, 1} | {s + 2 for s in range(nk) if s + 2 < nk})
    c_steps = sorted({0, 1, 2} | {s + 3 for s in range(nk) if s + 3 < nk})
    for tm in range(_cdiv(M, BM)):
        for tn in range(_cdiv(Ntot, BN)):
            m0, n0 = tm * BM, tn * BN
            for t in x_steps:
                kk = t * BK
                full = t >= 2 and kk + BK <= Ktot
                for i in range(4):
                    row = 32 * wave + 8 * i + (lane >> 3)
                    chunk = (lane & 7) ^ ((row ^ (row >> 2)) & 7)
                    m = np.minimum(m0 + row, M - 1)
                    off = (m * Ktot + 8 * chunk) * 2
                    if not full:
                        past = kk + 8 * chunk >= Ktot
                        off = np.where(past, off - (kk + 8 * chunk - (Ktot - 8)) * 2, off)
                    addr = 2 * kk + off
                    if (addr < 0).any() or (addr + 16 > M * Ktot * 2).any():
                        return f"In fetch of step {t}"
            for t in c_steps:
                kk = min(t * BK, (nk - 1) * BK)
                if mode == 0:
                    wrow = np.minimum(n0 + (p >> 1), d - 1)
                    ca = (wrow * k + kk + 32 * (p & 1)) >> 1
                    srow = np.minimum(n0 + e, d - 1)
                    blk = (srow * k + kk) >> 6
                else:
                    j = np.minimum(kk + (p >> 2), d - 1)
                    col = n0 + 32 * (p & 3)
                    ca = (j * k + np.where(col < k, col, k - 32)) >> 1
                    c0 = n0 + 64 * (e & 1)
                    blk = (np.minimum(kk + (e >> 1), d - 1) * k + np.where(c0 < k, c0, k - 64)) >> 6
                ca, blk = ca[cw], blk[sw]
                if (ca < 0).any() or (ca + 16 > d * k // 2).any():
                    return f"code fetch of step {t}"
                if dq:
                    q = (blk & ~3)[wave[sw] < 6]
                    if (q < 0).any() or (q + 4 > nb).any():
                        return f"int8-code fetch of step {t}"
                    if ((blk >> 8)[wave[sw] >= 6] >= ng).any():
                        return f"s2 fetch of step {t}"
                elif (blk < 0).any() or (blk >= nb).any():
                    return f"absmax fetch of step {t}"
    return None


SHAPES = [
    (256, 256, 300), (4096, 4096, 256), (256, 512, 300), (200, 320, 300),
    (384, 192, 17), (264, 128, 513), (8, 64, 2), (8, 64, 300), (72, 64, 40),
    (136, 576, 40), (2048, 11008, 256), (11008, 512, 256), (8, 128, 257),
    (16, 64, 256), (24, 192, 1),
]


@pytest.mark.parametrize("d,k,M", SHAPES)
@pytest.mark.parametrize("mode", [0, 1], ids=["fwd", "dx"])
@pytest.mark.parametrize("dq", [False, True], ids=["absmax", "dq"])
def test_gemm_fetches_stay_in_bounds(d, k, M, mode, dq):
    assert _fetches_in_bounds(d, k, M, mode, dq) is None


def test_model_catches_unsigned_clamp_wrap():
    # The clamp of a one-step contraction's prologue fetch, done in unsigned
    # 32-bit arithmetic, wraps to ~4 GB past the buffer: the model must see it.
    M, Ktot, kk = 2, 8, BK
    off = (1 * Ktot + 8 * 3) * 2
    wrapped = (off - (kk + 8 * 3 - (Ktot - 8)) * 2) % (1 << 32)
    assert 2 * kk + wrapped + 16 > M * Ktot * 2
    signed = off - (kk + 8 * 3 - (Ktot - 8)) * 2
    assert 0 <= 2 * kk + signed and 2 * kk + signed + 16 <= M * Ktot * 2
