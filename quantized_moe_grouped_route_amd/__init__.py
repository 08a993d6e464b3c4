"""Quantized MoE grouped GEMM for AMD Instinct MI355X (gfx950).

A thin Python binding over the C-ABI library libmoeq.so (include/moeq.h).
Each function here only checks and marshals its torch arguments (device
pointers, sizes, torch's current HIP stream) and calls the C entry point of
the same name; every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory and streams only.

If libmoeq.so is missing or cannot be loaded, every call raises: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoeq.so")

# Status codes and enums of include/moeq.h.
OK, EINVAL, EALIGN, EUNSUPPORTED, EHIP = 0, 1, 2, 3, 4
F16, BF16, F32, I32 = 1, 2, 3, 4
ACT = {"none": 0, "silu_mul": 1}
ACT_SILU_MUL_LIMIT = 2
AROW = {"token": 0, "sorted": 1}
SCHED = {"auto": 0, "decode": 1, "prefill": 2}
SF_LAYOUT = {"rows": 0, "quads": 1}
W_LAYOUT = {"rows": 0, "tiled": 1}

_DTYPE_CODE = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32, torch.int32: I32}

EXPORTS = ("moeq_last_error", "moeq_abi_version", "moe_route_prep_workspace_bytes",
           "moe_route_prep", "grouped_gemm_qint4", "grouped_gemm_qfp8_block",
           "grouped_gemm_qnvfp4", "moe_scatter_combine", "moe_quantize_int4",
           "moe_nvfp4_repack", "moe_sum_pairs", "moe_cast_bf16_to_f16", "moe_route_prep_noalloc")

# Fixed device scratch of moe_route_prep_noalloc per GPU (include/moeq.h).
ROUTE_NOALLOC_SCRATCH_BYTES = 1 << 20
# int32 counters of grouped_gemm_qnvfp4's optional work queue (include/moeq.h).
WORK_QUEUE_INTS = 16


def work_queue(device="cuda"):
    """A zeroed work queue for grouped_gemm_qnvfp4 (each call leaves it zero;
    calls that may overlap in time need their own)."""
    return torch.zeros(WORK_QUEUE_INTS, dtype=torch.int32, device=device)


class MoeqError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_lib = None


def lib():
    """The loaded C library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m quantized_moe_grouped_route_amd.build`")
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    sig = {
        "moeq_last_error": (C.c_char_p, []),
        "moeq_abi_version": (i32, []),
        "moe_route_prep_workspace_bytes": (sz, [i64, i32, i32]),
        "moe_route_prep": (i32, [vp, i64, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
        "moe_route_prep_noalloc": (i32, [vp, i64, i32, i32, vp, vp, vp, vp, vp]),
        "grouped_gemm_qint4": (i32, [vp, vp, i64, i32, vp, vp, vp, vp, i64, i32, i32, i64, i64,
                                     i32, i32, vp, i32, vp]),
        "grouped_gemm_qfp8_block": (i32, [vp, vp, i64, i32, vp, vp, vp, vp, i64, i32, i32, i64,
                                          i64, i32, vp, i32, vp]),
        "grouped_gemm_qnvfp4": (i32, [vp, i32, i64, i32, vp, i32, vp, i32, vp, vp, vp, i64, i32, i32, i64, i64,
                                      i32, C.c_float, vp, i32, vp, vp, i32, vp]),
        "moe_scatter_combine": (i32, [vp, i32, vp, vp, i64, i32, i64, i32, vp, vp]),
        "moe_quantize_int4": (i32, [vp, i32, i64, i64, vp, vp, vp]),
        "moe_nvfp4_repack": (i32, [vp, vp, i64, i64, i64, i32, i32, i32, vp, vp, vp]),
        "moe_sum_pairs": (i32, [vp, i32, vp, i64, i32, i64, i32, vp, vp]),
        "moe_cast_bf16_to_f16": (i32, [vp, i64, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def _check(fn: str, st: int):
    if st != OK:
        raise MoeqError(fn, st, lib().moeq_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _need(t, name, dtype=None, ndim=None):
    """Type, dtype, rank and contiguity of one tensor argument (where it
    lives is checked by _gpu, after every shape check)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _gpu(**tensors):
    """Every tensor argument (None: absent) must be in GPU memory."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")


def route_workspace_bytes(T: int, topk: int, E: int) -> int:
    return int(lib().moe_route_prep_workspace_bytes(T, topk, E))


def moe_route_prep(topk_ids, E: int, *, out=None, workspace=None):
    """Group the (token, slot) pairs by expert.

    topk_ids int32 [T][topk] on the GPU.  Returns (expert_offsets [E+1],
    sorted_pair_ids [P], pair_to_sorted [P], n_invalid [1]), all int32;
    `out` may supply these four tensors preallocated, `workspace` a uint8
    tensor of route_workspace_bytes(T, topk, E) bytes."""
    _need(topk_ids, "topk_ids", torch.int32, 2)
    T, k = topk_ids.shape
    P = T * k
    dev = topk_ids.device
    if out is None:
        out = (torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(P, dtype=torch.int32, device=dev),
               torch.empty(P, dtype=torch.int32, device=dev),
               torch.empty(1, dtype=torch.int32, device=dev))
    offs, srt, p2s, ninv = out
    for t, n, sz in ((offs, "expert_offsets", E + 1), (srt, "sorted_pair_ids", P),
                     (p2s, "pair_to_sorted", P), (ninv, "n_invalid", 1)):
        _need(t, n, torch.int32)
        if t.numel() < sz:
            raise ValueError(f"{n} needs {sz} elements")
    need = route_workspace_bytes(T, k, E)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _gpu(topk_ids=topk_ids, expert_offsets=offs, sorted_pair_ids=srt, pair_to_sorted=p2s, n_invalid=ninv,
         workspace=workspace)
    st = lib().moe_route_prep(_ptr(topk_ids), T, k, E, _ptr(offs), _ptr(srt), _ptr(p2s),
                              _ptr(ninv), _ptr(workspace), wsb, _stream())
    _check("moe_route_prep", st)
    return offs, srt, p2s, ninv


def moe_route_prep_noalloc(topk_ids, E: int, *, out):
    """moe_route_prep without a workspace: the library keeps the per-chunk
    counts in its fixed per-GPU device array (ROUTE_NOALLOC_SCRATCH_BYTES),
    so the call allocates nothing.  `out` supplies the four int32 output
    tensors (expert_offsets [E+1], sorted_pair_ids [P], pair_to_sorted [P],
    n_invalid [1]).  Calls that overlap in time on one GPU race."""
    _need(topk_ids, "topk_ids", torch.int32, 2)
    T, k = topk_ids.shape
    P = T * k
    offs, srt, p2s, ninv = out
    for t, n, sz in ((offs, "expert_offsets", E + 1), (srt, "sorted_pair_ids", P),
                     (p2s, "pair_to_sorted", P), (ninv, "n_invalid", 1)):
        _need(t, n, torch.int32)
        if t.numel() < sz:
            raise ValueError(f"{n} needs {sz} elements")
    _gpu(topk_ids=topk_ids, expert_offsets=offs, sorted_pair_ids=srt, pair_to_sorted=p2s, n_invalid=ninv)
    st = lib().moe_route_prep_noalloc(_ptr(topk_ids), T, k, E, _ptr(offs), _ptr(srt), _ptr(p2s), _ptr(ninv),
                                      _stream())
    _check("moe_route_prep_noalloc", st)
    return offs, srt, p2s, ninv


def _grouped_common(a, expert_offsets, sorted_pair_ids, a_row, P):
    _need(expert_offsets, "expert_offsets", torch.int32, 1)
    if sorted_pair_ids is not None:
        _need(sorted_pair_ids, "sorted_pair_ids", torch.int32, 1)
    E = expert_offsets.numel() - 1
    if P is None:
        P = sorted_pair_ids.numel() if sorted_pair_ids is not None else a.shape[0]
    return E, P, AROW[a_row]


def _out(out, P, n_out, dtype, dev):
    if out is None:
        return torch.empty(P, n_out, dtype=dtype, device=dev)
    _need(out, "out", dtype, 2)
    if out.shape[0] < P or out.shape[1] != n_out:
        raise ValueError(f"out must be [{P}][{n_out}], got {tuple(out.shape)}")
    return out


def grouped_gemm_qint4(a, a_scale, w, w_scale, expert_offsets, sorted_pair_ids, topk: int, *,
                       a_row="token", act="none", out_dtype=torch.float16, out=None, P=None,
                       sched="auto"):
    """W4A4 INT4 grouped GEMM: a uint8 [rows_a][K/2], a_scale f32 [rows_a],
    w uint8 [E][N][K/2], w_scale f32 [E][N].  Returns out [P][N] (act
    'none') or [P][N/2] ('silu_mul'); out_dtype torch.int32 gives the raw
    accumulators."""
    _need(a, "a", torch.uint8, 2)
    _need(a_scale, "a_scale", torch.float32, 1)
    _need(w, "w", torch.uint8, 3)
    _need(w_scale, "w_scale", torch.float32, 2)
    E, P, arow = _grouped_common(a, expert_offsets, sorted_pair_ids, a_row, P)
    En, N, Kh = w.shape
    K = 2 * Kh
    if En != E or a.shape[1] != Kh or tuple(w_scale.shape) != (E, N) or a_scale.numel() != a.shape[0]:
        raise ValueError("inconsistent INT4 operand shapes")
    out = _out(out, P, N // 2 if act == "silu_mul" else N, out_dtype, a.device)
    _gpu(a=a, a_scale=a_scale, w=w, w_scale=w_scale, expert_offsets=expert_offsets,
         sorted_pair_ids=sorted_pair_ids, out=out)
    st = lib().grouped_gemm_qint4(_ptr(a), _ptr(a_scale), a.shape[0], arow, _ptr(w), _ptr(w_scale),
                                  _ptr(expert_offsets), _ptr(sorted_pair_ids), P, topk, E, N, K,
                                  ACT[act], _DTYPE_CODE[out_dtype], _ptr(out), SCHED[sched],
                                  _stream())
    _check("grouped_gemm_qint4", st)
    return out


def grouped_gemm_qfp8_block(a, a_scale, w, w_scale, expert_offsets, sorted_pair_ids, topk: int, *,
                            a_row="token", out_dtype=torch.bfloat16, out=None, P=None,
                            sched="auto"):
    """FP8 e4m3 block-scaled grouped GEMM: a uint8 [rows_a][K] (e4m3 bits),
    a_scale f32 [K/128][rows_a], w uint8 [E][N][K], w_scale f32
    [E][N/128][K/128].  Returns out [P][N]."""
    _need(a, "a", torch.uint8, 2)
    _need(a_scale, "a_scale", torch.float32, 2)
    _need(w, "w", torch.uint8, 3)
    _need(w_scale, "w_scale", torch.float32, 3)
    E, P, arow = _grouped_common(a, expert_offsets, sorted_pair_ids, a_row, P)
    En, N, K = w.shape
    if (En != E or a.shape[1] != K or tuple(a_scale.shape) != (K // 128, a.shape[0])
            or tuple(w_scale.shape) != (E, N // 128, K // 128)):
        raise ValueError("inconsistent FP8 operand shapes")
    out = _out(out, P, N, out_dtype, a.device)
    _gpu(a=a, a_scale=a_scale, w=w, w_scale=w_scale, expert_offsets=expert_offsets,
         sorted_pair_ids=sorted_pair_ids, out=out)
    st = lib().grouped_gemm_qfp8_block(_ptr(a), _ptr(a_scale), a.shape[0], arow, _ptr(w),
                                       _ptr(w_scale), _ptr(expert_offsets), _ptr(sorted_pair_ids),
                                       P, topk, E, N, K, _DTYPE_CODE[out_dtype], _ptr(out),
                                       SCHED[sched], _stream())
    _check("grouped_gemm_qfp8_block", st)
    return out


def grouped_gemm_qnvfp4(x, w, w_sf, w_gscale, expert_offsets, sorted_pair_ids, topk: int, *,
                        a_row="token", act="none", limit=None, pair_weights=None,
                        out_dtype=torch.bfloat16, out=None, P=None, sched="auto", work_queue=None):
    """NVFP4 W4A16 grouped GEMM: x bf16 or f16 [rows_a][K] (f16: dequant and
    MFMA in binary16, megamoe_rm.cu's fp16 activations), w uint8 [E][N][K/2]
    (row-major) or [E][N/16][K/64][16][32] (tiled)
    (E2M1), w_sf uint8 [E][N][K/16] (UE4M3, row-major), uint8 [E][K/64][N][4]
    (K-quad-major, faster for the tiled schedule) or int32 [E][N][K/64] (four
    UE4M3 per word, block 4g+j in bits 8j..8j+7: the row-major bytes), w_gscale
    f32 [E].  Returns out [P][N] (act 'none') or [P][N/2] ('silu_mul';
    with `limit`, the clamped SwiGLU of megamoe_rm.cu's fc1_rm).
    pair_weights (f32, T*topk values, e.g. topk_weights): megamoe_rm.cu's
    fc2_rm epilogue, out row p = w[p] * y of pair p, in pair order.
    work_queue (int32, WORK_QUEUE_INTS zeros, see work_queue()): the tiled
    schedule then balances its tiles through atomic counters in it."""
    _need(x, "x", (torch.bfloat16, torch.float16), 2)
    _need(w, "w", torch.uint8)
    if w.dim() == 5 and tuple(w.shape[3:]) == (16, 32):
        w_tiled = True
        En, N, K = w.shape[0], 16 * w.shape[1], 64 * w.shape[2]
    elif w.dim() == 3:
        w_tiled = False
        En, N, K = w.shape[0], w.shape[1], 2 * w.shape[2]
    else:
        raise ValueError("w must be [E][N][K/2] or [E][N/16][K/64][16][32]")
    if isinstance(w_sf, torch.Tensor) and w_sf.dtype == torch.int32 and w_sf.dim() == 3:
        _need(w_sf, "w_sf", torch.int32, 3)
        w_sf = w_sf.view(torch.uint8)                   # [E][N][K/64] words -> [E][N][K/16] bytes
    _need(w_sf, "w_sf", torch.uint8)
    quads = w_sf.dim() == 4
    _need(w_gscale, "w_gscale", torch.float32, 1)
    E, P, arow = _grouped_common(x, expert_offsets, sorted_pair_ids, a_row, P)
    sf_shape = (E, K // 64, N, 4) if quads else (E, N, K // 16)
    if En != E or x.shape[1] != K or tuple(w_sf.shape) != sf_shape or w_gscale.numel() != E:
        raise ValueError("inconsistent NVFP4 operand shapes")
    if limit is not None and act != "silu_mul":
        raise ValueError("limit applies to act 'silu_mul' only")
    act_code = ACT[act] if limit is None else ACT_SILU_MUL_LIMIT
    if pair_weights is not None:
        _need(pair_weights, "pair_weights", torch.float32)
        if sorted_pair_ids is None or pair_weights.numel() != sorted_pair_ids.numel():
            raise ValueError("pair_weights needs sorted_pair_ids and one weight per pair")
        if P < sorted_pair_ids.numel():
            # rows are written at pair ids, which run up to sorted_pair_ids.numel() - 1
            raise ValueError("with pair_weights, P must be at least the number of pairs")
    if work_queue is not None:
        _need(work_queue, "work_queue", torch.int32, 1)
        if work_queue.numel() < WORK_QUEUE_INTS:
            raise ValueError(f"work_queue needs {WORK_QUEUE_INTS} int32")
    out = _out(out, P, N // 2 if act == "silu_mul" else N, out_dtype, x.device)
    _gpu(x=x, w=w, w_sf=w_sf, w_gscale=w_gscale, expert_offsets=expert_offsets,
         sorted_pair_ids=sorted_pair_ids, pair_weights=pair_weights, work_queue=work_queue, out=out)
    st = lib().grouped_gemm_qnvfp4(_ptr(x), _DTYPE_CODE[x.dtype], x.shape[0], arow, _ptr(w),
                                   W_LAYOUT["tiled" if w_tiled else "rows"], _ptr(w_sf),
                                   SF_LAYOUT["quads" if quads else "rows"], _ptr(w_gscale),
                                   _ptr(expert_offsets), _ptr(sorted_pair_ids), P, topk, E, N, K,
                                   act_code, 0.0 if limit is None else float(limit), _ptr(pair_weights),
                                   _DTYPE_CODE[out_dtype], _ptr(out), _ptr(work_queue), SCHED[sched], _stream())
    _check("grouped_gemm_qnvfp4", st)
    return out


def moe_scatter_combine(y, pair_to_sorted, topk_weights, *, out_dtype=None, out=None):
    """out[t] = sum_j topk_weights[t, j] * y[pair_to_sorted[t*k+j]] over the
    routed slots of token t, fp32 in slot order, one rounding."""
    _need(y, "y", (torch.float16, torch.bfloat16, torch.float32), 2)
    _need(pair_to_sorted, "pair_to_sorted", torch.int32, 1)
    _need(topk_weights, "topk_weights", torch.float32, 2)
    T, k = topk_weights.shape
    N = y.shape[1]
    if pair_to_sorted.numel() != T * k:
        raise ValueError("pair_to_sorted must have T*topk entries")
    if y.shape[0] < T * k:
        raise ValueError("y must have at least T*topk rows (sorted positions index into it)")
    out_dtype = out_dtype or y.dtype
    if out is None:
        out = torch.empty(T, N, dtype=out_dtype, device=y.device)
    _need(out, "out", out_dtype, 2)
    if tuple(out.shape) != (T, N):
        raise ValueError(f"out must be [{T}][{N}], got {tuple(out.shape)}")
    _gpu(y=y, pair_to_sorted=pair_to_sorted, topk_weights=topk_weights, out=out)
    st = lib().moe_scatter_combine(_ptr(y), _DTYPE_CODE[y.dtype], _ptr(pair_to_sorted),
                                   _ptr(topk_weights), T, k, N, _DTYPE_CODE[out_dtype], _ptr(out),
                                   _stream())
    _check("moe_scatter_combine", st)
    return out


def moe_sum_pairs(y_pairs, pair_to_sorted, T: int, topk: int, *, out_dtype=None, out=None):
    """out[t] = sum_j y_pairs[t*topk + j] over the slots of token t that have
    an expert (pair_to_sorted >= 0), fp32 in slot order, one rounding: the
    combine that follows grouped_gemm_qnvfp4(..., pair_weights=...)."""
    _need(y_pairs, "y_pairs", (torch.float16, torch.bfloat16, torch.float32), 2)
    _need(pair_to_sorted, "pair_to_sorted", torch.int32, 1)
    N = y_pairs.shape[1]
    if pair_to_sorted.numel() != T * topk or y_pairs.shape[0] < T * topk:
        raise ValueError("pair_to_sorted needs T*topk entries and y_pairs T*topk rows")
    out_dtype = out_dtype or y_pairs.dtype
    if out is None:
        out = torch.empty(T, N, dtype=out_dtype, device=y_pairs.device)
    _need(out, "out", out_dtype, 2)
    if tuple(out.shape) != (T, N):
        raise ValueError(f"out must be [{T}][{N}], got {tuple(out.shape)}")
    _gpu(y_pairs=y_pairs, pair_to_sorted=pair_to_sorted, out=out)
    st = lib().moe_sum_pairs(_ptr(y_pairs), _DTYPE_CODE[y_pairs.dtype], _ptr(pair_to_sorted), T, topk, N,
                             _DTYPE_CODE[out_dtype], _ptr(out), _stream())
    _check("moe_sum_pairs", st)
    return out


def cast_bf16_to_f16(x, *, out=None):
    """bf16 tensor -> binary16 tensor of the same shape, each value rounded
    once to nearest even (exact for magnitudes in [2^-14, 65504]); `out` may
    be x viewed as float16 (in place) or a separate contiguous tensor."""
    _need(x, "x", torch.bfloat16)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float16, device=x.device)
    _need(out, "out", torch.float16)
    if out.numel() != x.numel():
        raise ValueError("out must have as many elements as x")
    _gpu(x=x, out=out)
    st = lib().moe_cast_bf16_to_f16(_ptr(x), x.numel(), _ptr(out), _stream())
    _check("moe_cast_bf16_to_f16", st)
    return out


def quantize_int4_rows(x, *, q=None, scale=None):
    """Per-row symmetric int4 codes of x [rows][K] (f16/bf16/f32): returns
    (q uint8 [rows][K/2], scale f32 [rows]), s = amax/7, codes
    rne(x * 7/amax) clamped to [-8, 7], packed low nibble first."""
    _need(x, "x", (torch.float16, torch.bfloat16, torch.float32), 2)
    rows, K = x.shape
    if q is None:
        q = torch.empty(rows, K // 2, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(rows, dtype=torch.float32, device=x.device)
    _need(q, "q", (torch.uint8,), 2)
    _need(scale, "scale", (torch.float32,), 1)
    if tuple(q.shape) != (rows, K // 2) or tuple(scale.shape) != (rows,):
        raise ValueError("quantize_int4_rows: q must be [rows][K/2] and scale [rows]")
    _gpu(x=x, q=q, scale=scale)
    st = lib().moe_quantize_int4(_ptr(x), _DTYPE_CODE[x.dtype], rows, K, _ptr(q), _ptr(scale), _stream())
    _check("moe_quantize_int4", st)
    return q, scale


def nvfp4_repack(w, sf_swizzled, *, swap_halves: bool, sf_layout="rows", w_layout="rows", w_out=None,
                 sf_out=None):
    """Convert NVFP4 expert weights from the in-place layout of megamoe_rm.cu
    (w uint8 [E][N][K/2]; sf_swizzled uint8 [E][N*K/16] in 128x4 tiles;
    swap_halves for a w13 stored up rows first) to grouped_gemm_qnvfp4's
    layout.  Returns (w_out [E][N][K/2] for w_layout 'rows' or
    [E][N/16][K/64][16][32] for 'tiled', sf_out [E][N][K/16] for sf_layout
    'rows' or [E][K/64][N][4] for 'quads')."""
    _need(w, "w", torch.uint8, 3)
    _need(sf_swizzled, "sf_swizzled", torch.uint8, 2)
    E, N, Kh = w.shape
    K = 2 * Kh
    if tuple(sf_swizzled.shape) != (E, N * K // 16):
        raise ValueError("sf_swizzled must be [E][N*K/16]")
    w_shape = (E, N // 16, K // 64, 16, 32) if w_layout == "tiled" else (E, N, Kh)
    if w_out is None:
        w_out = torch.empty(w_shape, dtype=torch.uint8, device=w.device)
    sf_shape = (E, K // 64, N, 4) if sf_layout == "quads" else (E, N, K // 16)
    if sf_out is None:
        sf_out = torch.empty(sf_shape, dtype=torch.uint8, device=w.device)
    _need(w_out, "w_out", torch.uint8)
    _need(sf_out, "sf_out", torch.uint8)
    if tuple(w_out.shape) != w_shape or tuple(sf_out.shape) != sf_shape:
        raise ValueError(f"w_out must be {w_shape} and sf_out {sf_shape}")
    _gpu(w=w, sf_swizzled=sf_swizzled, w_out=w_out, sf_out=sf_out)
    st = lib().moe_nvfp4_repack(_ptr(w), _ptr(sf_swizzled), E, N, K, int(bool(swap_halves)),
                                W_LAYOUT[w_layout], SF_LAYOUT[sf_layout], _ptr(w_out), _ptr(sf_out),
                                _stream())
    _check("moe_nvfp4_repack", st)
    return w_out, sf_out
