"""Seeded synthetic inputs for the quantized MoE grouped GEMM workloads.

This module only draws random numbers and stores them in the byte formats the
path consumes.  It contains none of the path's arithmetic (no decoding, no
routing table, no contraction, no combine): both the CPU oracle and the GPU
path read exactly the arrays made here.

Conventions (shared input formats, not arithmetic):
  * 4-bit codes (INT4, E2M1) are packed two per byte, element 2b in the low
    nibble of byte b.  Uniform codes are drawn as uniform random bytes.
  * bf16 tensors are carried as their uint16 bit patterns (made by torch's
    float32 -> bfloat16 cast, round to nearest even).
  * FP8 is OCP e4m3fn, carried as uint8 bit patterns.
  * Each workload draws from ``np.random.SeedSequence(seed).spawn(9)``, one
    stream per role (ROLE_* below), so one role can change size without
    perturbing the others.
"""
from __future__ import annotations

import numpy as np

ROLE_ROUTING, ROLE_LOGITS, ROLE_ACT, ROLE_ACT_SCALE = 0, 1, 2, 3
ROLE_W1, ROLE_S1, ROLE_W2, ROLE_S2, ROLE_GSCALE = 4, 5, 6, 7, 8


def streams(seed: int):
    """Nine independent generators, one per role."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(9)]


# ----------------------------------------------------------------- routing
def distinct_uniform_ids(rng, T: int, k: int, E: int) -> np.ndarray:
    """k distinct expert ids per token, uniform over [0, E)."""
    if T == 0:
        return np.zeros((0, k), np.int32)
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def uniform_ids_with_repeats(rng, T: int, k: int, E: int) -> np.ndarray:
    """k expert ids per token, independent uniform draws (repeats allowed)."""
    return rng.integers(0, E, size=(T, k), dtype=np.int32)


def zipf_ids(rng, T: int, k: int, E: int, s: float = 1.1, n_zero: int = 8) -> np.ndarray:
    """k distinct ids per token drawn without replacement with p(e) proportional
    to rank(e)^-s, rank a seeded permutation of the experts; n_zero seeded
    experts get p = 0 so that some experts receive no rows.

    Sampling without replacement by Gumbel top-k (equivalent to successive
    draws proportional to p)."""
    rank = rng.permutation(E)
    p = (rank + 1.0) ** (-s)
    if n_zero:
        p[rng.choice(E, size=n_zero, replace=False)] = 0.0
    assert k <= int((p > 0).sum())
    with np.errstate(divide="ignore"):
        logp = np.log(p)
    keys = logp[None, :] + rng.gumbel(size=(T, E))
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def softmax_weights(rng, T: int, k: int) -> np.ndarray:
    """Router weights: softmax over k logits drawn N(0,1), float32."""
    z = rng.standard_normal((T, k))
    z = np.exp(z - z.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


# ----------------------------------------------------------------- values
def uniform_bytes(rng, shape) -> np.ndarray:
    """Uniform random bytes: every packed 4-bit code uniform over its 16 codes."""
    n = int(np.prod(shape, dtype=np.int64))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def uniform_f32(rng, shape, lo: float, hi: float) -> np.ndarray:
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def scale_bytes(rng, shape, lo: int = 0x30, hi: int = 0x47) -> np.ndarray:
    """UE4M3 block-scale bytes, uniform over the codes lo..hi inclusive
    (0x30..0x47 is 0.5 .. 3.75)."""
    return rng.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest even, torch's cast) as uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(rng, shape) -> np.ndarray:
    return bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))


def e4m3_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3fn bits via torch's cast (round to nearest even).
    The caller clamps to +-448 first: the cast does not saturate."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def fp8_quant_1x128(x: np.ndarray):
    """Per-row, per-128-column quantization of x [M][K] (input recipe):
    scale = amax/448 (1 where amax is 0), q = e4m3(clamp(x/scale, +-448)).
    Returns q [M][K] uint8 and scales laid out [K/128][M] (M contiguous)."""
    M, K = x.shape
    assert K % 128 == 0
    xb = x.reshape(M, K // 128, 128).astype(np.float32)
    amax = np.abs(xb).max(axis=2)
    sc = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = e4m3_bits(np.clip(xb / sc[:, :, None], -448.0, 448.0).reshape(M, K))
    return q, np.ascontiguousarray(sc.T)


def fp8_quant_128x128(w: np.ndarray):
    """Per 128x128 block quantization of w [N][K] (input recipe as above).
    Returns q [N][K] uint8 and scales [N/128][K/128]."""
    N, K = w.shape
    assert N % 128 == 0 and K % 128 == 0
    wb = w.reshape(N // 128, 128, K // 128, 128).astype(np.float32)
    amax = np.abs(wb).max(axis=(1, 3))
    sc = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = e4m3_bits(np.clip(wb / sc[:, None, :, None], -448.0, 448.0).reshape(N, K))
    return q, sc


# ----------------------------------------------------------------- problems
def int4_moe(seed: int, T: int, E: int, k: int, N: int, K: int, *, routing="distinct",
             fc2_rows: int = 0, N2: int = 0, K2: int = 0):
    """W4A4 INT4 grouped problem: activations int4 [T][K/2] bytes with per-token
    scales U[0.005,0.05]; weights int4 [E][N][K/2] with per-channel scales
    U[0.005,0.05]; ids (distinct uniform, or 'repeat' for independent draws),
    softmax top-k weights.  With fc2_rows > 0 also a second (SORTED-row)
    problem: int4 rows [fc2_rows][K2/2] with per-row scales and weights
    [E][N2][K2/2] with per-channel scales."""
    r = streams(seed)
    ids = (distinct_uniform_ids if routing == "distinct" else uniform_ids_with_repeats)(
        r[ROLE_ROUTING], T, k, E)
    d = dict(topk_ids=ids, topk_weights=softmax_weights(r[ROLE_LOGITS], T, k),
             a=uniform_bytes(r[ROLE_ACT], (T, K // 2)),
             a_scale=uniform_f32(r[ROLE_ACT_SCALE], (T,), 0.005, 0.05),
             w=uniform_bytes(r[ROLE_W1], (E, N, K // 2)),
             w_scale=uniform_f32(r[ROLE_S1], (E, N), 0.005, 0.05),
             T=T, E=E, k=k, N=N, K=K)
    if fc2_rows:
        w2 = uniform_bytes(r[ROLE_W2], (E, N2, K2 // 2))
        w2_scale = uniform_f32(r[ROLE_S2], (E, N2), 0.005, 0.05)
        d.update(w2=w2, w2_scale=w2_scale,
                 a2=uniform_bytes(r[ROLE_W2], (fc2_rows, K2 // 2)),
                 a2_scale=uniform_f32(r[ROLE_S2], (fc2_rows,), 0.005, 0.05),
                 N2=N2, K2=K2)
    return d


def fp8_block(seed: int, M: int, N: int, K: int, E: int = 1, *, T: int = 0, k: int = 1):
    """FP8 e4m3 block-scaled problem.  Dense (E=1, T=0): A [M][K] and B [1][N][K]
    from N(0,1), quantized per 1x128 (A) and per 128x128 (B).  Routed (T>0):
    A holds T token rows, ids distinct uniform over E experts."""
    r = streams(seed)
    rows = M if T == 0 else T
    a, sa = fp8_quant_1x128(r[ROLE_ACT].standard_normal((rows, K), dtype=np.float32))
    ws, sbs = [], []
    for _ in range(E):
        q, s = fp8_quant_128x128(r[ROLE_W1].standard_normal((N, K), dtype=np.float32))
        ws.append(q)
        sbs.append(s)
    d = dict(a=a, a_scale=sa, w=np.stack(ws), w_scale=np.stack(sbs), M=rows, N=N, K=K, E=E)
    if T == 0:
        d.update(topk_ids=np.zeros((rows, 1), np.int32), topk_weights=np.ones((rows, 1), np.float32),
                 T=rows, k=1)
    else:
        d.update(topk_ids=distinct_uniform_ids(r[ROLE_ROUTING], T, k, E),
                 topk_weights=softmax_weights(r[ROLE_LOGITS], T, k), T=T, k=k)
    return d


def fp8_moe(seed: int, T: int, E: int, k: int, N: int, K: int):
    """FP8 e4m3 block-scaled MoE projection for decode (DeepSeek-V3 style
    scales): A [T][K] from N(0,1) quantized per 1x128; W [E][N][K] with e4m3
    codes uniform over all non-NaN bytes, generated for the routed experts
    only (the others are never read and stay zero); w_scale [E][N/128][K/128]
    uniform in [0.5, 1.5] / 448; ids distinct uniform over E."""
    r = streams(seed)
    ids = distinct_uniform_ids(r[ROLE_ROUTING], T, k, E)
    a, sa = fp8_quant_1x128(r[ROLE_ACT].standard_normal((T, K), dtype=np.float32))
    w = np.zeros((E, N, K), np.uint8)
    for e in np.unique(ids[(ids >= 0) & (ids < E)]):
        codes = uniform_bytes(r[ROLE_W1], (N, K))
        codes[(codes & 0x7F) == 0x7F] ^= 1          # no NaN codes
        w[e] = codes
    w_scale = (r[ROLE_S1].uniform(0.5, 1.5, (E, N // 128, K // 128)) / 448.0).astype(np.float32)
    return dict(a=a, a_scale=sa, w=w, w_scale=w_scale, topk_ids=ids,
                topk_weights=softmax_weights(r[ROLE_LOGITS], T, k), T=T, E=E, k=k, N=N, K=K, M=T)


def nvfp4_moe(seed: int, T: int, E: int, k: int, H: int, I: int, *, routing="distinct",
              scale_lo: int = 0x30, scale_hi: int = 0x47):
    """NVFP4 W4A16 MoE layer: x [T][H] bf16 from N(0,1); w1 (gate rows [0,I) then
    up rows [I,2I)) [E][2I][H/2] and w2 [E][H][I/2] with uniform E2M1 codes;
    UE4M3 scales per 16 along K, bytes uniform in [scale_lo, scale_hi];
    global scales g1 = 2^-9 U[0.75,1.25], g2 = 2^-7 U[0.75,1.25].
    routing: 'distinct' | 'zipf' | 'repeat'."""
    r = streams(seed)
    if routing == "distinct":
        ids = distinct_uniform_ids(r[ROLE_ROUTING], T, k, E)
    elif routing == "zipf":
        ids = zipf_ids(r[ROLE_ROUTING], T, k, E)
    else:
        ids = uniform_ids_with_repeats(r[ROLE_ROUTING], T, k, E)
    d = dict(topk_ids=ids, topk_weights=softmax_weights(r[ROLE_LOGITS], T, k),
             x=normal_bf16(r[ROLE_ACT], (T, H)),
             w1=uniform_bytes(r[ROLE_W1], (E, 2 * I, H // 2)),
             s1=scale_bytes(r[ROLE_S1], (E, 2 * I, H // 16), scale_lo, scale_hi),
             w2=uniform_bytes(r[ROLE_W2], (E, H, I // 2)),
             s2=scale_bytes(r[ROLE_S2], (E, H, I // 16), scale_lo, scale_hi),
             T=T, E=E, k=k, H=H, I=I)
    g = r[ROLE_GSCALE]
    d["g1"] = (2.0 ** -9 * g.uniform(0.75, 1.25, E)).astype(np.float32)
    d["g2"] = (2.0 ** -7 * g.uniform(0.75, 1.25, E)).astype(np.float32)
    return d


# RMS of an int4 code uniform over [-8, 7]: sqrt(mean of c^2) = sqrt(21.5)
INT4_RMS = 4.637


def int4_chain(seed: int, T: int, E: int, k: int, H: int, I: int):
    """The full W4A4 layer from fp16 activations: x [T][H] fp16 from N(0,1)
    times a per-row factor U[0.5, 2]; gate+up weights [E][2I][H/2] and down
    weights [E][H][I/2], int4 codes uniform over [-8, 7].  Per-channel
    weight scales are U[0.5, 1.5] / (sqrt(K) * INT4_RMS), so each GEMM keeps
    its input's magnitude and h and y stay well inside fp16 (the U[0.005,
    0.05] scales of the raw-int4 workloads grow activations about tenfold per
    GEMM on random codes, which overflows fp16 by the second one).  Distinct
    uniform ids, softmax top-k weights."""
    r = streams(seed)
    x = r[ROLE_ACT].standard_normal((T, H), dtype=np.float32)
    x *= r[ROLE_ACT_SCALE].uniform(0.5, 2.0, (T, 1)).astype(np.float32)
    s1 = 1.0 / (np.sqrt(H) * INT4_RMS)
    s2 = 1.0 / (np.sqrt(I) * INT4_RMS)
    return dict(x=x.astype(np.float16), topk_ids=distinct_uniform_ids(r[ROLE_ROUTING], T, k, E),
                topk_weights=softmax_weights(r[ROLE_LOGITS], T, k),
                w=uniform_bytes(r[ROLE_W1], (E, 2 * I, H // 2)),
                w_scale=uniform_f32(r[ROLE_S1], (E, 2 * I), 0.5 * s1, 1.5 * s1),
                w2=uniform_bytes(r[ROLE_W2], (E, H, I // 2)),
                w2_scale=uniform_f32(r[ROLE_S2], (E, H), 0.5 * s2, 1.5 * s2),
                T=T, E=E, k=k, H=H, I=I, N=2 * I, K=H)


def nvfp4_stored_weights(seed: int, E: int, N: int, K: int):
    """NVFP4 expert weights as another runtime stores them (megamoe_rm.cu's
    in-place layout): w [E][N][K/2] uniform E2M1 code bytes and the UE4M3
    scales of each expert as one run of N*K/16 bytes, sf [E][N*K/16].  The
    scale bytes are drawn iid, so drawing them directly in the stored byte
    order gives the same distribution as drawing a [N][K/16] matrix and
    rearranging it; no layout arithmetic happens here."""
    r = streams(seed)
    return dict(w=uniform_bytes(r[ROLE_W1], (E, N, K // 2)),
                sf=scale_bytes(r[ROLE_S1], (E, N * K // 16)), E=E, N=N, K=K)


# ------------------------------------------------------ the measured workloads
# Sizes of the measured workloads (seed = 1000 + index).
WORKLOADS = {
    0: dict(name="w4a4_int4_tiny", kind="int4", T=64, E=4, k=2, N=256, K=256),
    1: dict(name="fp8_block_dense_1024x4096x7168", kind="fp8", M=1024, N=4096, K=7168),
    2: dict(name="nvfp4_w4a16_decode_T8", kind="nvfp4", T=8, E=256, k=8, H=7168, I=2048,
            routing="distinct"),
    3: dict(name="nvfp4_w4a16_prefill_T4096_zipf", kind="nvfp4", T=4096, E=256, k=8, H=7168,
            I=2048, routing="zipf"),
    4: dict(name="w4a4_int4_mixtral_T8192", kind="int4", T=8192, E=8, k=2, H=4096, I=14336),
    # per-row int4 quantization of the Mixtral-sized W4A4 layer's FC1 output h
    # (T*k rows of I fp16)
    5: dict(name="int4_quantize_rows_16384x14336_f16", kind="quant", rows=16384, K=14336),
    # the FP8 block-scaled kernel under routing: one 8-token decode step of a
    # DeepSeek-V3-shaped expert projection (gate+up, N = 2I = 4096, K = H)
    6: dict(name="fp8_block_moe_decode_T8", kind="fp8", T=8, E=256, k=8, N=4096, K=7168),
    # one-shot repack of the NVFP4 decode workload's gate+up weights (E=256 experts of
    # 2I = 4096 rows, K = H = 7168) from the up-first, 128x4-swizzled-scale
    # layout of megamoe_rm.cu
    7: dict(name="nvfp4_repack_w13_E256_N4096_K7168", kind="repack", E=256, N=4096, K=7168, swap=1),
    # the complete Mixtral-sized W4A4 layer from fp16 activations:
    # per-token int4 of x, FC1 (SiLU), per-row int4 of h, FC2, combine
    8: dict(name="w4a4_int4_chain_mixtral_T8192", kind="int4chain", T=8192, E=8, k=2, H=4096, I=14336),
    # the same layer for one 8-token decode step: 16 routed rows over the 8
    # experts, so the GEMMs stream the weights (HBM-bound)
    9: dict(name="w4a4_int4_chain_mixtral_decode_T8", kind="int4chain", T=8, E=8, k=2, H=4096, I=14336),
}


def workload(idx: int):
    """Materialize workload idx on the host (large ones take seconds and GBs)."""
    c = WORKLOADS[idx]
    seed = 1000 + idx
    if idx == 0:
        return int4_moe(seed, c["T"], c["E"], c["k"], c["N"], c["K"])
    if idx == 1:
        return fp8_block(seed, c["M"], c["N"], c["K"])
    if idx in (2, 3):
        return nvfp4_moe(seed, c["T"], c["E"], c["k"], c["H"], c["I"], routing=c["routing"])
    if idx == 4:
        # FC1: tokens [T][H] x gate_up [E][2I][H]; FC2: synthetic SORTED int4 rows
        # [T*k][I] with per-row scales x down [E][H][I].
        return int4_moe(seed, c["T"], c["E"], c["k"], 2 * c["I"], c["H"],
                        fc2_rows=c["T"] * c["k"], N2=c["H"], K2=c["I"])
    if idx == 5:
        r = streams(seed)
        x = r[ROLE_ACT].standard_normal((c["rows"], c["K"]), dtype=np.float32)
        x *= r[ROLE_ACT_SCALE].uniform(0.1, 10.0, (c["rows"], 1)).astype(np.float32)
        return dict(x=x.astype(np.float16))
    if idx == 6:
        return fp8_moe(seed, c["T"], c["E"], c["k"], c["N"], c["K"])
    if idx == 7:
        return nvfp4_stored_weights(seed, c["E"], c["N"], c["K"])
    if idx in (8, 9):
        return int4_chain(seed, c["T"], c["E"], c["k"], c["H"], c["I"])
    raise KeyError(idx)
