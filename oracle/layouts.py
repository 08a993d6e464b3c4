"""Weight layout conversion for the NVFP4 path (TEST INFRASTRUCTURE ONLY; see
the package docstring).

megamoe_rm.cu (the header comment of the file and its scale_off function)
describes the NVFP4 MoE layout vLLM's FlashInfer CUTLASS backend keeps after
processing, which that kernel reads in place:
  * w13 per expert is [2I][K/2] bytes with the UP projection in rows 0..I-1 and
    the GATE projection in rows I..2I-1 (the library's SILU_MUL layout is the
    other way round: gate rows first);
  * the UE4M3 block scales of a [R][C] scale matrix (C = K/16 blocks per row)
    are stored in tiles of 128 rows x 4 block columns, 512 bytes per tile.
    Tiles follow each other row-block major: tile (R//128, C//4) order.
    Inside a tile, row r (of the 128) is split as r = 32q + i, q in 0..3,
    i in 0..31.  Its 4 bytes for block columns 4j..4j+3 sit at
    16*i + 4*q + (c % 4).
The repack below turns that layout into the library's linear one
([R][C] row-major scales, gate rows first when asked), one-shot, before the
GEMMs run: a load-time conversion instead of a second set of GEMM kernels.

The library also reads a second scale layout of its own, "K-quad major":
for each group of 4 consecutive block columns (a quad, 64 values of K),
the 4 scale bytes of every row, rows consecutive: s_q[e, j, n, i] =
s[e, n, 4j + i], stored [E][C/4][R][4].  One K step of 64 then finds the
scales of many consecutive rows in one contiguous run.

And a weight layout of its own, "tiled": each expert's [R][K/2] code bytes
cut into blocks of 16 rows x 32 bytes (64 values of K), a 16-row group's
blocks consecutive along K: byte (n, b) at
((n // 16) * (K/64) + b // 32) * 512 + (n % 16) * 32 + b % 32.
"""
import numpy as np


def scale_swizzle_offset(r, c, C: int):
    """Byte offset of the scale of row r, block column c in a swizzled [R][C]
    scale matrix (megamoe_rm.cu, scale_off).  r, c may be integer arrays.
    Needs C % 4 == 0; the matrix needs R % 128 == 0."""
    r = np.asarray(r, np.int64)
    c = np.asarray(c, np.int64)
    tile = (r // 128) * (C // 4) + (c // 4)          # row block, then column quad
    within = (r % 32) * 16 + ((r // 32) % 4) * 4 + (c % 4)
    return tile * 512 + within


def unswizzle_scales(s_swz: np.ndarray, R: int, C: int) -> np.ndarray:
    """[.., R*C] swizzled bytes (any leading expert dims) -> [.., R, C] linear."""
    if R % 128 or C % 4:
        raise ValueError("the 128x4 swizzle needs R % 128 == 0 and C % 4 == 0")
    lead = s_swz.shape[:-1]
    src = np.asarray(s_swz).reshape(lead + (R * C,))
    rr, cc = np.meshgrid(np.arange(R), np.arange(C), indexing="ij")
    return src[..., scale_swizzle_offset(rr, cc, C)]


def swizzle_scales(s_lin: np.ndarray) -> np.ndarray:
    """[.., R, C] linear -> [.., R*C] swizzled bytes (the inverse of
    unswizzle_scales; used to build inputs in the pages' layout)."""
    lead, (R, C) = s_lin.shape[:-2], s_lin.shape[-2:]
    if R % 128 or C % 4:
        raise ValueError("the 128x4 swizzle needs R % 128 == 0 and C % 4 == 0")
    out = np.empty(lead + (R * C,), s_lin.dtype)
    rr, cc = np.meshgrid(np.arange(R), np.arange(C), indexing="ij")
    out[..., scale_swizzle_offset(rr, cc, C)] = s_lin
    return out


def quads_from_rows(s_lin: np.ndarray) -> np.ndarray:
    """[.., R, C] row-major scales -> [.., C/4, R, 4] K-quad-major bytes."""
    lead, (R, C) = s_lin.shape[:-2], s_lin.shape[-2:]
    if C % 4:
        raise ValueError("the quad layout needs C % 4 == 0")
    q = np.asarray(s_lin).reshape(lead + (R, C // 4, 4))
    return np.ascontiguousarray(np.swapaxes(q, -3, -2))


def rows_from_quads(s_q: np.ndarray) -> np.ndarray:
    """[.., C/4, R, 4] K-quad-major -> [.., R, C] row-major (the inverse)."""
    lead, (Q, R, four) = s_q.shape[:-3], s_q.shape[-3:]
    assert four == 4
    return np.ascontiguousarray(np.swapaxes(np.asarray(s_q), -3, -2)).reshape(lead + (R, 4 * Q))


def tiles_from_rows(w: np.ndarray) -> np.ndarray:
    """[.., R, K/2] row-major codes -> [.., R/16, K/64, 16, 32] tiled bytes."""
    lead, (R, KB) = w.shape[:-2], w.shape[-2:]
    if R % 16 or KB % 32:
        raise ValueError("the tiled layout needs R % 16 == 0 and K % 64 == 0")
    t = np.asarray(w).reshape(lead + (R // 16, 16, KB // 32, 32))
    return np.ascontiguousarray(np.swapaxes(t, -3, -2))


def rows_from_tiles(w_t: np.ndarray) -> np.ndarray:
    """[.., R/16, K/64, 16, 32] tiled -> [.., R, K/2] row-major (the inverse)."""
    lead, (G, Q, sixteen, thirtytwo) = w_t.shape[:-4], w_t.shape[-4:]
    assert sixteen == 16 and thirtytwo == 32
    return np.ascontiguousarray(np.swapaxes(np.asarray(w_t), -3, -2)).reshape(lead + (16 * G, 32 * Q))


def repack_nvfp4(w: np.ndarray, s_swz: np.ndarray, swap_halves: bool, out_layout: str = "rows",
                 w_layout: str = "rows"):
    """Weights w [E][R][K/2] and swizzled scales s_swz [E][R*K/16] in the
    megamoe_rm.cu layout -> (w_lin [E][R][K/2], s_lin [E][R][K/16]) in the
    library's layout.  swap_halves: the matrix is a w13 (up rows first); the
    output puts the gate rows [R/2, R) first, then the up rows [0, R/2).
    out_layout 'rows' returns scales [E][R][K/16], 'quads' [E][K/64][R][4];
    w_layout 'rows' returns codes [E][R][K/2], 'tiled' [E][R/16][K/64][16][32]."""
    E, R, KB = w.shape
    C = KB // 8                                        # K/16 blocks = (K/2 bytes) / 8
    s_lin = unswizzle_scales(s_swz, R, C)
    if swap_halves:
        if R % 2:
            raise ValueError("swap_halves needs an even row count")
        h = R // 2
        order = np.concatenate([np.arange(h, R), np.arange(0, h)])
        w_out, s_out = w[:, order, :], s_lin[:, order, :]
    else:
        w_out, s_out = w.copy(), s_lin
    if w_layout == "tiled":
        w_out = tiles_from_rows(w_out)
    elif w_layout != "rows":
        raise ValueError(w_layout)
    if out_layout == "quads":
        return w_out, quads_from_rows(s_out)
    if out_layout != "rows":
        raise ValueError(out_layout)
    return w_out, s_out
