"""Lane-level CPU model of the float 3D hard tile (tile3d_lut in
euler_characteristic_curves_amd/csrc/ecc_hard.hip).  Test infrastructure: it
models the kernel's arithmetic so that the tile logic can be checked against
the oracle on the CPU; it is not used by the library and computes nothing the
tests take as a reference.

For every tile (a chunk of 64*VEC columns, TY rows of one wave, a range of
planes) it forms the keys as the kernel does, as LDS byte addresses
bin * 4C + 4 * (lane mod C) (C interleaved histogram copies), including the
edge keys (the values just outside the chunk, carrying the copy offset of the
lane that uses them, 0 or 63), trash keys for cells outside the grid, the
lane-neighbour moves, the four row sequences of the telescoped decomposition
and its weight formula ((d >> 24) of the neighbour differences), and adds the
weights into a model of the LDS histogram.  Binning follows the kernel's
bucket table (one threshold per bucket, or up to 8 scanned) or its binary
search, with the same float32 bucket map (the 2^23-biased fma rounding).
Loads: 'full' chunks, 'scalar' (element loads of unaligned rows, clamped
columns) and 'partial' (vector loads of aligned rows past the row end: lanes
past it carry trash keys).
"""
from fractions import Fraction

import numpy as np

F32 = np.float32


def running_max(tau):
    return np.maximum.accumulate(tau.astype(np.float32))


def build_lut(R, n):
    """The bucket table exactly as build_lut computes it (float32 arithmetic)."""
    H = R.size
    lo, hi = F32(R[0]), F32(R[H - 1])
    ok = H >= 2 and np.isfinite(lo) and np.isfinite(hi) and hi > lo
    mul = add = F32(0)
    if ok:
        mul = F32(F32(n - 1) / F32(hi - lo))
        add = F32(-lo * mul)
        ok = mul > 0 and np.isfinite(mul) and np.isfinite(add)
    if not ok:
        return None

    # The kernel evaluates fma(v, mul, add + 2^23) in float32: between 2^23
    # and 2^24 float32 holds exactly the integers, so the fma's single
    # rounding is round-half-even of v * mul + add_b - 2^23; med3 then clamps
    # to [0, n - 1] (NaN to 0) and the bucket is read from the bit pattern.
    bias = 2.0 ** 23
    add_b = F32(np.float64(add) + bias)   # float32 add + 2^23 (exact in float64)

    def bucket(v):
        v = float(v)
        if np.isnan(v):
            return 0
        if np.isinf(v):
            return n - 1 if (v > 0) == (float(mul) > 0) and mul != 0 else 0
        # v * mul is exact in float64 (24 + 24 bits); the sum rounds at most
        # once more, which can only move the final rounding on an exact
        # float64 tie, where the exact rational decides instead
        x = v * float(mul) + float(add_b) - bias
        if x - np.floor(x) == 0.5:
            x = Fraction(v) * Fraction(float(mul)) + Fraction(float(add_b)) - Fraction(bias)
        return min(max(int(round(x)), 0), n - 1)

    bk = [bucket(r) for r in R]
    # per-bucket counts
    worst = 1
    for k in range(H):
        if k == 0 or bk[k - 1] < bk[k]:
            c = 1
            while c <= 8 and k + c < H and bk[k + c] == bk[k]:
                c += 1
            worst = max(worst, c)
    mode = 1 if worst == 1 else (2 if worst <= 8 else 0)
    if mode == 0:
        return ('search', None, bucket)
    table = {}
    for k in range(H + 1):
        bprev = bk[k - 1] if k > 0 else -1
        b = bk[k] if k < H else n - 1
        for j in range(bprev + 1, b + 1):
            here = k < H and j == b
            if mode == 1:
                table[j] = (R[k] if here else np.inf, k)
            else:
                cnt = 0
                if here:
                    cnt = 1
                    while cnt <= 8 and k + cnt < H and bk[k + cnt] == b:
                        cnt += 1
                table[j] = (cnt, k)
    return ('lut1' if mode == 1 else 'lut2', table, bucket)


def make_key(R, lut, C):
    H = R.size
    kind, table, bucket = lut if lut else ('search', None, None)

    def bin_of(v):
        if kind == 'lut1':
            thr, base = table[bucket(v)]
            return base + (1 if v > thr else 0)
        if kind == 'lut2':
            cnt, base = table[bucket(v)]
            return base + sum(1 for i in range(cnt) if R[base + i] < v)
        # search: number of R_k below v with a power-of-two walk
        k, top = 0, 1
        while top * 2 <= H:
            top *= 2
        step = top
        while step > 0:
            if k + step <= H and R[k + step - 1] < v:
                k += step
            step //= 2
        return k

    def key(v, lane):
        return bin_of(v) * 4 * C + 4 * (lane % C)

    return key, kind


def emulate(grid, tau, TY=4, VEC=4, C=32, TZ=2, loads='auto', force_kind=None, partial_ty=None):
    """ECC of grid at tau as the tiles compute it.  partial_ty: tile height of
    the partial chunks of aligned rows (the kernel runs them two rows at a
    time, and full chunks TY rows at a time); None uses TY for every chunk."""
    nz, ny, nx = grid.shape
    H = tau.size
    R = running_max(tau)
    lut = build_lut(R, 2 * H + 2)
    key, kind = make_key(R, lut, C)
    if force_kind:
        kind = force_kind
    trash_bin = H
    CH = 64 * VEC
    hist = np.zeros((H + 1) * C * 4, dtype=np.int64)   # indexed by byte address / 4 ... use dict by address
    hist = {}

    def add(addr, w):
        hist[addr] = hist.get(addr, 0) + w

    aligned = (nx * 4) % (VEC * 4) == 0
    ntx = (nx + CH - 1) // CH
    for xb in range(0, ntx * CH, CH):
        full = aligned and xb + CH <= nx
        mode = 'full' if full else ('partial' if (aligned and loads == 'partial') else 'scalar')
        has_l, has_r = xb > 0, xb + CH < nx
        lim = min(nx - 1 - xb, CH - 1)
        ty = partial_ty if (mode == 'partial' and partial_ty) else TY
        for ys in range(0, ny, ty):
            for zs in range(0, nz, TZ):
                ze = min(zs + TZ, nz)
                tile(grid, key, C, ty, VEC, xb, ys, zs, ze, has_l, has_r, lim, mode, trash_bin, add)
    # histogram by bin
    hb = np.zeros(H + 1, dtype=np.int64)
    for addr, w in hist.items():
        hb[addr // (4 * C)] += w
    return np.cumsum(hb[:H]), kind


def tile(grid, key, C, TY, VEC, xb, ys, zs, ze, has_l, has_r, lim, mode, trash_bin, add):
    nz, ny, nx = grid.shape
    CH = 64 * VEC
    lanes = np.arange(64)

    def trash(lane):
        return trash_bin * 4 * C + 4 * (lane % C)

    def row_keys(z, r):
        """keys[64][VEC] of row ys+r of plane z (invalid plane/row -> trash)."""
        ok = z < nz and ys + r < ny
        zc = min(z, nz - 1)
        yc = min(ys + r, ny - 1)
        k = np.empty((64, VEC), dtype=np.int64)
        for l in range(64):
            for j in range(VEC):
                c = VEC * l + j
                if not ok:
                    k[l, j] = trash(l)
                    continue
                if mode == 'full':
                    k[l, j] = key(grid[zc, yc, xb + c], l)
                elif mode == 'scalar':
                    cc = min(c, lim)
                    kk = key(grid[zc, yc, xb + cc], l)
                    k[l, j] = kk if c <= lim else trash(l)
                else:  # partial: lanes wholly past the row end carry trash
                    if xb + VEC * l < nx:
                        k[l, j] = key(grid[zc, yc, xb + c], l)
                    else:
                        k[l, j] = trash(l)
        return k

    def edge_keys(z, r):
        """(left key as lane 0 uses it, right key as lane 63 uses it) of row ys+r."""
        ok = z < nz
        zc = min(z, nz - 1)
        yc = min(ys + r, ny - 1)
        row_ok = ys + r < ny
        L = key(grid[zc, yc, xb - 1], 0) if (ok and has_l and row_ok) else trash(0)
        Rr = key(grid[zc, yc, xb + CH], 63) if (ok and has_r and row_ok) else trash(63)
        return L, Rr

    def tele(s, left, right, sign):
        # s: [64][VEC] keys; left/right: edge values for lanes 0 / 63
        flat = s.reshape(-1)
        nxt = np.append(flat[1:], right)
        prv = np.insert(flat[:-1], 0, left)
        for i in range(flat.size):
            d = int(flat[i] - nxt[i])
            dp = int(prv[i] - flat[i])
            sh = lambda x: -1 if x < 0 else 0  # arithmetic >> 24 of |x| < 2^24
            w = (sh(dp) - sh(d)) if sign > 0 else (sh(d) - sh(dp))
            add(int(flat[i]), w)

    A = [row_keys(zs, r) for r in range(TY + 1)]
    AE = [edge_keys(zs, r) for r in range(TY + 1)]
    for z in range(zs, ze):
        B = [row_keys(z + 1, r) for r in range(TY + 1)]
        BE = [edge_keys(z + 1, r) for r in range(TY + 1)]
        for r in range(TY):
            if ys + r >= ny:
                continue
            s1 = A[r]
            s2 = np.maximum(A[r], A[r + 1])
            s3 = np.maximum(A[r], B[r])
            s4 = np.maximum(s2, np.maximum(B[r], B[r + 1]))
            l1, r1 = AE[r]
            l2, r2 = max(AE[r][0], AE[r + 1][0]), max(AE[r][1], AE[r + 1][1])
            l3, r3 = max(AE[r][0], BE[r][0]), max(AE[r][1], BE[r][1])
            l4 = max(l2, max(BE[r][0], BE[r + 1][0]))
            r4 = max(r2, max(BE[r][1], BE[r + 1][1]))
            tele(s1, l1, r1, 1)
            tele(s2, l2, r2, -1)
            tele(s3, l3, r3, -1)
            tele(s4, l4, r4, 1)
        A, AE = B, BE


