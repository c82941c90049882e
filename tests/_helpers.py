"""Test-side helpers: decoding the documented code layouts, mask comparison with the
near-tie rule, and the parity metrics."""
import numpy as np


def _qk_map():
    # byte ((t*4 + s)*64 + lane)*16 + e  <->  row 32t + r, channel 64g + 16s + e  (lane = 32g + r)
    m = np.empty((64, 128), np.int64)
    for row in range(64):
        for ch in range(128):
            t, r, g, s, e = row // 32, row % 32, ch // 64, (ch % 64) // 16, ch % 16
            m[row, ch] = ((t * 4 + s) * 64 + (g * 32 + r)) * 16 + e
    return m


def _v_map():
    # byte ((dt*2 + e/16)*64 + lane)*16 + e%16  <->  channel 32dt + r of token
    # 32(e/16) + 8((e%16)/4) + 4g + e%4
    m = np.empty((64, 128), np.int64)
    for dt in range(4):
        for lane in range(64):
            g, r = lane // 32, lane % 32
            for e in range(32):
                tok = 32 * (e // 16) + 8 * ((e % 16) // 4) + 4 * g + e % 4
                m[tok, 32 * dt + r] = ((dt * 2 + e // 16) * 64 + lane) * 16 + e % 16
    return m


QK_MAP = _qk_map()
V_MAP = _v_map()


def decode_qk_codes(blocks):
    """[Nb, 8192] int8 code blocks -> [Nb*64, 128] rows."""
    b = np.asarray(blocks)
    return b[:, QK_MAP].reshape(-1, 128)


def decode_v_codes(blocks):
    b = np.asarray(blocks)
    return b[:, V_MAP].reshape(-1, 128)


def mask_mismatch(gpu_idx, ora_idx, score_rows, tol=1e-5):
    """Rows whose kept sets differ; raises if a difference is not a near-tie.

    score_rows: oracle fp64 scores of the same rows. A difference is allowed only when
    every swapped-in and swapped-out block's scores lie within tol of each other.
    """
    bad = []
    for r in range(len(ora_idx)):
        G, O = set(gpu_idx[r].tolist()), set(ora_idx[r].tolist())
        if G == O:
            continue
        assert len(G) == len(O) == len(ora_idx[r])
        inn = [score_rows[r][j] for j in G - O]
        out = [score_rows[r][j] for j in O - G]
        gap = max(out) - min(inn)
        assert gap < tol, "row %d: mask differs by more than a near-tie (gap %.3g)" % (r, gap)
        bad.append(r)
    return bad


def cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def decode_w8a8_tiles(buf, RT, K):
    """Block-major 32 x 128 INT8 code tiles -> [32*RT][K] rows.

    Tile (kb, rt) sits at byte (kb*RT + rt)*4096; byte (s*64 + lane)*16 + e of a tile holds
    row 32rt + lane%32, channel 128kb + 64(lane/32) + 16s + e."""
    KB = K // 128
    a = np.asarray(buf).view(np.int8)[: KB * RT * 4096].reshape(KB, RT, 4, 2, 32, 16)  # kb, rt, s, g, r, e
    return a.transpose(1, 4, 0, 3, 2, 5).reshape(RT * 32, K)
