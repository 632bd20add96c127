"""A lane-by-lane CPU model of the staged-window kernel for the stride-2, 4x4
transposed convolution (tconv_halo_kernel), checked against the oracle (CPU
only).

The model restates, in numpy, what each lane of that kernel does: the
buffer-to-LDS copies (global offset per lane, LDS unit per lane, the XOR
swizzle of the weight rows and the nine-unit window pitch), the per-wave
wait counts and the workgroup barrier, the MFMA operand reads, the 32x32x16
operand and result lane layouts, the bias-initialised accumulators, the
bf16 packing with its lane swaps and 8-lane row shifts, and the store offsets.
Copies stay pending per instruction until a wait lets them land, so a read of
a buffer that still has a copy in flight fails the run.  It checks that every
LDS and global index stays in range, that every output element is written
exactly once, and that the result equals the oracle exactly on integer data.
Two planted mistakes (the read-side swizzle dropped; a wait that leaves a
weight copy in flight) must fail it.

The constants below restate the kernel's; a test reads them back from the
kernel source, so a change there fails here until the model follows.
"""
import os
import re

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "cnn_convolution_conv2d_amd",
                   "csrc", "transposed.hip")

BK, WIN_H, WIN_W, POS_H, POS_W, CO, PITCH = 64, 10, 34, 8, 32, 64, 9
WAVES, ROWS, XCOPIES = 8, 4, 48
WUNITS = 4 * CO * 8
XUNITS = WIN_H * WIN_W * PITCH
OOB = 0x7FFFFFF0
LANE = np.arange(64)


def xj(t):
    """Window copies of the next block issued in step t: j in [xj(t), xj(t+1))."""
    return 2 * t if t < 2 else t + 2


def permlane32_swap(x, y):
    xn, yn = x.copy(), y.copy()
    xn[32:] = y[:32]
    yn[:32] = x[32:]
    return xn, yn


def permlane16_swap(x, y):
    xn, yn = x.copy(), y.copy()
    xn[16:32], xn[48:64] = y[0:16], y[32:48]
    yn[0:16], yn[32:48] = x[16:32], x[48:64]
    return xn, yn


def row_shift(old, src, shift, bank_mask):
    """DPP row_shr:shift (row_shl for a negative shift) under a bank mask,
    bound_ctrl off: lanes outside the mask or without a source keep old."""
    out = old.copy()
    for l in range(64):
        s = l - shift
        if (bank_mask >> ((l % 16) // 4)) & 1 and 0 <= s < 64 and s // 16 == l // 16:
            out[l] = src[s]
    return out


def run_model(N, Cin, H, W, Cout, P, OP, relu, seed, read_swizzle=True, wait3=1):
    rng = np.random.default_rng(seed)
    x = rng.integers(-3, 4, size=(N, Cin, H, W)).astype(np.float64)
    w = rng.integers(-3, 4, size=(Cin, Cout, 4, 4)).astype(np.float64)
    b = rng.integers(-5, 6, size=Cout).astype(np.float64)
    yref, _ = oracle.conv_transpose2d(x, w, b, 2, P, OP, 1, 1, relu=relu)
    Ho, Wo = yref.shape[2], yref.shape[3]
    xg = x.transpose(0, 2, 3, 1).reshape(-1)                 # NHWC
    wpk = w.transpose(1, 2, 3, 0).reshape(-1)                # packed [Cout][4][4][Cin]
    y = np.full(N * Ho * Wo * Cout, np.nan)
    written = np.zeros(y.size, np.int64)

    def gload(buf, off):
        if off == OOB:
            return np.zeros(8)
        assert off % 16 == 0 and 0 <= off and off + 16 <= buf.size * 2, off
        return buf[off // 2:off // 2 + 8]

    lo = P // 2 - 1
    nbu = ((Ho + 1) // 2 + POS_H - 1) // POS_H
    nbv = ((Wo + 1) // 2 + POS_W - 1) // POS_W
    ncb = (Cout + CO - 1) // CO
    nblk = (Cin + BK - 1) // BK
    for item in range(N * nbu * nbv * ncb):
        it = item
        cb = it % ncb
        it //= ncb
        bv = it % nbv
        it //= nbv
        bu, n = it % nbu, it // nbu
        co0, u0, v0 = cb * CO, bu * POS_H, bv * POS_W
        ih0, iw0 = u0 + lo, v0 + lo
        wl = np.full((2, WUNITS, 8), np.nan)
        xl = np.full((2, XUNITS, 8), np.nan)
        pend = {wv: [] for wv in range(WAVES)}   # per wave: copy instructions in issue order

        def stage_w(buf, blk, t):
            c0, jh, jw = blk * BK, t >> 1, t & 1
            for wave in range(WAVES):
                for m in range(4):
                    i = wave + WAVES * m
                    ins = []
                    for lane in range(64):
                        row = 8 * i + (lane >> 3)
                        p, col = row >> 6, row & 63
                        piece = (lane & 7) ^ ((col >> 1) & 7)
                        kh = (((p >> 1) + P) & 1) + 2 * jh
                        kw = (((p & 1) + P) & 1) + 2 * jw
                        co, ci = co0 + col, c0 + 8 * piece
                        off = ((co * 16 + kh * 4 + kw) * Cin + ci) * 2 if co < Cout and ci < Cin else OOB
                        assert i * 64 + lane < WUNITS
                        ins.append(("w", buf, i * 64 + lane, gload(wpk, off).copy()))
                    pend[wave].append(ins)

        def stage_x(buf, blk, j0, j1):
            c0 = blk * BK
            for wave in range(WAVES):
                for j in range(j0, j1):
                    base = min(64 * (wave + WAVES * j), XUNITS - 64)
                    ins = []
                    for lane in range(64):
                        s = base + lane
                        wp, slot = s // PITCH, s % PITCH
                        ih, iw, ci = ih0 + wp // WIN_W, iw0 + wp % WIN_W, c0 + 8 * slot
                        ok = slot < 8 and ci < Cin and 0 <= ih < H and 0 <= iw < W
                        off = (((n * H + ih) * W + iw) * Cin + ci) * 2 if ok else OOB
                        assert s < XUNITS
                        ins.append(("x", buf, s, gload(xg, off).copy()))
                    pend[wave].append(ins)

        def wait(keep):
            """Every wave's copies but its `keep` youngest land (loads complete
            in order); the barrier that follows makes them everyone's."""
            for wv in range(WAVES):
                q = pend[wv]
                landed, pend[wv] = q[:len(q) - keep], q[len(q) - keep:]
                for ins in landed:
                    for kind, buf, u, v in ins:
                        (wl if kind == "w" else xl)[buf, u] = v

        waves = []
        acc = {}
        for wave in range(WAVES):
            p = wave & 3
            ph_h, ph_w, r0 = p >> 1, p & 1, ROWS * (wave >> 2)
            bh, bw = (ph_h + P) >> 1, (ph_w + P) >> 1
            tapo = [(r0 + bh - (t >> 1) - lo) * WIN_W + (bw - (t & 1) - lo) for t in range(4)]
            waves.append((ph_h, ph_w, r0, p, tapo, 2 * (u0 + r0) + ph_h < Ho))
            for i in range(2):
                a0 = np.zeros((16, 64))
                for q in range(4):
                    for e in range(4):
                        co = co0 + 32 * i + 8 * q + 4 * (LANE >> 5) + e
                        a0[4 * q + e] = np.where(co < Cout, b[np.minimum(co, Cout - 1)], 0.0)
                for r in range(ROWS):
                    acc[wave, i, r] = a0.copy()

        stage_x(0, 0, 0, 6)
        stage_w(0, 0, 0)
        for blk in range(nblk):
            more = blk + 1 < nblk
            for t in range(4):
                wait(0 if t == 0 or not more else (wait3 if t == 3 else 2))
                if t < 3:
                    stage_w((t + 1) & 1, blk, t + 1)
                elif more:
                    stage_w(0, blk + 1, 0)
                if more:
                    stage_x((blk + 1) & 1, blk + 1, xj(t), xj(t + 1))
                for wv in range(WAVES):
                    for kind, buf, _, _ in (e for ins in pend[wv] for e in ins):
                        assert not (kind == "w" and buf == (t & 1)), "weights read with a copy into them in flight"
                        assert not (kind == "x" and buf == (blk & 1)), "window read with a copy into it in flight"
                wc, xc = wl[t & 1], xl[blk & 1]
                for wave, (ph_h, ph_w, r0, p, tapo, act) in enumerate(waves):
                    if not act:
                        continue
                    frow, half = LANE & 31, LANE >> 5
                    sw = (frow >> 1) & 7 if read_swizzle else 0
                    for ks in range(4):
                        q = 2 * ks + half
                        A = [wc[(p * CO + 32 * i + frow) * 8 + (q ^ sw)] for i in range(2)]
                        B = []
                        for r in range(ROWS):
                            idx = (tapo[t] + r * WIN_W + frow) * PITCH + q
                            assert idx.min() >= 0 and idx.max() < XUNITS
                            B.append(xc[idx])
                        assert not any(np.isnan(v).any() for v in A + B), "operand read before its copy landed"
                        for i in range(2):
                            Am = np.zeros((32, 16))        # lane l: row l % 32, k 8*(l//32) .. +7
                            for l in range(64):
                                Am[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = A[i][l]
                            for r in range(ROWS):
                                Bm = np.zeros((16, 32))    # lane l: column l % 32, k 8*(l//32) .. +7
                                for l in range(64):
                                    Bm[8 * (l // 32):8 * (l // 32) + 8, l % 32] = B[r][l]
                                D = Am @ Bm
                                a = acc[wave, i, r]
                                for qq in range(4):
                                    for e in range(4):
                                        a[4 * qq + e] += D[8 * qq + 4 * (LANE >> 5) + e, LANE % 32]
        assert all(not v for v in pend.values())

        for wave, (ph_h, ph_w, r0, p, tapo, act) in enumerate(waves):
            if not act:
                continue
            if Cout % 8 == 0:
                co = co0 + ((LANE >> 4) & 1) * 16 + (LANE >> 5) * 8 + np.where(LANE & 8, 32, 0)
                for r in range(ROWS):
                    oh = 2 * (u0 + r0 + r) + ph_h

                    def pack(a):
                        v = np.maximum(a, 0) if relu else a
                        pk = [[np.stack([v[4 * q + 2 * k], v[4 * q + 2 * k + 1]], 1) for k in range(2)]
                              for q in range(4)]
                        r8 = [[None] * 4 for _ in range(2)]
                        for pr in range(2):
                            for k in range(2):
                                r8[pr][k], r8[pr][2 + k] = permlane32_swap(pk[2 * pr][k], pk[2 * pr + 1][k])
                        out = [[None] * 4, [None] * 4]
                        for d in range(4):
                            out[0][d], out[1][d] = permlane16_swap(r8[0][d], r8[1][d])
                        return out

                    o0, o1 = pack(acc[wave, 0, r]), pack(acc[wave, 1, r])
                    for h in range(2):
                        ra = [row_shift(o0[h][d], o1[h][d], 8, 0xC) for d in range(4)]
                        rb = [row_shift(o1[h][d], o0[h][d], -8, 0x3) for d in range(4)]
                        owa = 2 * (v0 + 16 * h + (LANE & 7)) + ph_w
                        for ow, reg in ((owa, ra), (owa + 16, rb)):
                            for l in range(64):
                                if oh < Ho and ow[l] < Wo and co[l] < Cout:
                                    off = ((n * Ho + oh) * Wo + ow[l]) * Cout + co[l]
                                    assert off % 8 == 0 and off + 8 <= y.size
                                    y[off:off + 8] = np.concatenate([reg[d][l] for d in range(4)])
                                    written[off:off + 8] += 1
            else:
                ow = 2 * (v0 + (LANE & 31)) + ph_w
                for i in range(2):
                    for q in range(4):
                        co = co0 + 32 * i + 8 * q + 4 * (LANE >> 5)
                        for r in range(ROWS):
                            oh = 2 * (u0 + r0 + r) + ph_h
                            a = acc[wave, i, r]
                            for l in range(64):
                                if oh < Ho and ow[l] < Wo and co[l] < Cout:
                                    off = ((n * Ho + oh) * Wo + ow[l]) * Cout + co[l]
                                    v = a[4 * q:4 * q + 4, l]
                                    y[off:off + 4] = np.maximum(v, 0) if relu else v
                                    written[off:off + 4] += 1
    assert (written == 1).all(), "every output element written exactly once"
    return y.reshape(N, Ho, Wo, Cout).transpose(0, 3, 1, 2), yref


CASES = [
    (2, 32, 9, 11, 48, 1, 0),      # several row tiles, ragged columns, a partial channel group
    (1, 32, 5, 6, 36, 0, 0),       # padding 0; Cout % 8 != 0 (the 8-byte store path)
    (2, 96, 4, 3, 8, 3, 0),        # padding 3; half of the second channel block past Cin
    (1, 192, 9, 30, 72, 2, 1),     # three channel blocks; two channel groups; output padding
]


def test_constants_match_the_kernel():
    src = open(SRC).read()

    def const(name):
        m = re.search(r"constexpr int " + name + r" = (\d+);", src)
        assert m, name
        return int(m.group(1))

    def pair(a, b):
        m = re.search(r"constexpr int " + a + r" = (\d+), " + b + r" = (\d+)", src)
        assert m, a
        return int(m.group(1)), int(m.group(2))

    assert (const("kThBK"), const("kThCo"), const("kThPitch"), const("kThXCopies")) == (BK, CO, PITCH, XCOPIES)
    assert pair("kThWin", "kTwWin") == (WIN_H, WIN_W)
    assert pair("kThPos", "kTwPos") == (POS_H, POS_W)
    m = re.search(r"constexpr int kThThreads = (\d+),", src)
    assert m and int(m.group(1)) == 64 * WAVES


@pytest.mark.parametrize("k", range(len(CASES)))
def test_model_equals_oracle(k):
    y, yref = run_model(*CASES[k], relu=bool(k % 2), seed=k)
    np.testing.assert_array_equal(y, yref)


def test_model_catches_a_dropped_read_swizzle():
    y, yref = run_model(*CASES[0], relu=False, seed=7, read_swizzle=False)
    assert not np.array_equal(y, yref)


def test_model_catches_a_short_wait():
    with pytest.raises(AssertionError, match="in flight"):
        run_model(*CASES[3], relu=False, seed=8, wait3=2)
