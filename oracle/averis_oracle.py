"""CPU oracle for the Averis hot path -- TEST INFRASTRUCTURE, not product code.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark may import
this module.  The HIP library never calls it and shares no code, table or constant with it.

What it computes is the mean-residual split before blockwise FP4 quantization of
"The Curse and Blessing of Mean Bias in FP4-Quantized LLM Training" (arXiv 2603.10444).
Pages cited below, by key:

  [rainbus]    "均值偏置的诅咒与祝福：FP4量化大语言模型训练" explainer (paper.rainbus.top)
  [paperlayer] "The Curse and Blessing of Mean Bias in FP4-Quantized LLM Training",
               source-linked summary of v2 (paperlayer.ai)
  [gist]       German summary of the same paper (gist.science), "Technische Zusammenfassung"
  [chatpaper]  v1 abstract (chatpaper.ai)

Precision: every step the GPU takes in fp32 (residual, Hadamard butterflies, scale arithmetic,
element scaling) is done here in IEEE fp32 with one rounding per operation (numpy float32
ufuncs never contract to FMA).  Reductions over the token axis and the GEMMs run in fp64 on
dequantized values, i.e. they are the exact products up to fp64 rounding.

Readings where the pages are silent (all listed again in the design notes):
  * block formats: NVFP4-style = 16-element blocks, E4M3 block scale, fp32 tensor decode scale
    s_dec = amax / (6 * 448); MXFP4 = 32-element blocks, E8M0 scale 2^(floor(log2 amax) - 2)
    (OCP MX v1.0 rule).  The pages only name E2M1 and "scale set by the block max".
  * rounding is round-to-nearest-even everywhere; E2M1 saturates at 6, E4M3 at 448.
  * element scaling multiplies by the fp32 reciprocal of the block decode scale.
  * the sign of a non-zero-block element that rounds to 0 is kept (code 0x8);
    blocks whose scale is zero (or whose decode scale underflows fp32's normal range) get
    all-zero codes.
  * each operand is quantized in blocks along its own GEMM's reduction axis, so X_R and D_R are
    each quantized twice (K = features for fwd/dX, K = tokens for dW), W twice (K = m, K = n).
  * every layout is zero-padded along K, after subtraction, to a multiple of 256 elements.
  * the mean vector is quantized along its length with its own tensor scale; the optional
    16x16 Hadamard rotates every operand along its reduction axis (the mean too), and the
    weight-gradient rank-one term undoes the mean's rotation exactly.
  * dW keeps only the two terms the pages keep (cross terms dropped).
"""
from __future__ import annotations

import numpy as np

NVFP4 = 1
MXFP4 = 2
BLOCK = {NVFP4: 16, MXFP4: 32}
KPAD = 256  # storage padding multiple along K (zero elements after the logical length)

F32 = np.float32


# --------------------------------------------------------------------------------------------
# Number formats.  [rainbus] 前置知识 / FP4量化: FP4 is E2M1 (2 exponent bits, 1 mantissa bit);
# 块量化: one scale per block, set by the block's largest magnitude.
# --------------------------------------------------------------------------------------------

def e2m1_value(code):
    """Value of a 4-bit E2M1 code: bit 3 sign, bits 2:1 exponent (bias 1), bit 0 mantissa.

    Exponent field 0 is subnormal (0 or 0.5); otherwise 2^(e-1) * (1 + m/2).
    """
    code = np.asarray(code, dtype=np.int64)
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(code & 8, -mag, mag)


def e2m1_encode(v):
    """Round fp32 values to the nearest E2M1 code, ties to the even code, saturating at 6.

    The magnitude grid is {0, .5, 1, 1.5, 2, 3, 4, 6}; midpoints between neighbours decide,
    and a midpoint goes to the neighbour whose code is even.  The sign bit is the sign of v.
    """
    v = np.asarray(v, dtype=F32)
    a = np.abs(v)
    c = np.zeros(v.shape, dtype=np.uint8)
    c[a > 0.25] = 1      # 0.25 is the 0 | 0.5 midpoint: goes to code 0
    c[a >= 0.75] = 2     # 0.75: 0.5 | 1 midpoint: code 2
    c[a > 1.25] = 3      # 1.25: 1 | 1.5 midpoint: code 2
    c[a >= 1.75] = 4     # 1.75: 1.5 | 2: code 4
    c[a > 2.5] = 5       # 2.5: 2 | 3: code 4
    c[a >= 3.5] = 6      # 3.5: 3 | 4: code 6
    c[a > 5.0] = 7       # 5: 4 | 6: code 6; everything above 5 saturates to 6
    c |= (np.signbit(v).astype(np.uint8) << 3)
    return c


def e4m3_value(code):
    """Value of a non-negative E4M3 (fn variant) code: bias 7, no infinities, 0x7F is NaN."""
    code = np.asarray(code, dtype=np.int64)
    e = (code >> 3) & 15
    m = code & 7
    return np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                    np.ldexp(1.0 + m / 8.0, e - 7))


def e4m3_encode(v):
    """Round non-negative finite fp32 values to E4M3, nearest-even, saturating at 448 (0x7E).

    Normal range step is 2^(floor(log2 v) - 3); below 2^-6 the subnormal step is 2^-9.
    """
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(v)
    flog = np.maximum(ex - 1, -6)                 # binade of the quantum (clamped to subnormal)
    qexp = flog - 3
    q = np.rint(np.ldexp(v, -qexp))               # exact scaling, then round half to even
    val = np.minimum(np.ldexp(q, qexp), 448.0)    # satfinite
    _, ev = np.frexp(val)
    E = np.where(val >= 2.0 ** -6, (ev - 1) + 7, 0)
    M = np.where(E > 0, np.rint((np.ldexp(val, -(ev - 1)) - 1.0) * 8.0),
                 np.rint(np.ldexp(val, 9)))
    code = (E.astype(np.int64) << 3) | M.astype(np.int64)
    return np.where(val == 0.0, 0, code).astype(np.uint8)


def mx_scale_exponent(amax):
    """E8M0 shared exponent of an MXFP4 block: floor(log2 amax) - 2, clamped to [-127, 127].

    2 is the largest exponent of E2M1 (6 = 1.5 * 2^2).  amax == 0 gives -127.
    """
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(a)
    E = (ex - 1) - 2
    E = np.where(a == 0.0, -127, E)
    return np.clip(E, -127, 127).astype(np.int64)


# --------------------------------------------------------------------------------------------
# Stochastic rounding of E2M1 (an option: the pages round to nearest).  Random bits come from
# Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw, "Parallel random
# numbers: as easy as 1, 2, 3" (SC 2011): ten rounds of two 32 x 32 -> 64-bit multiplies on a
# 4-word counter under a 2-word key, the key bumped by the Weyl constants between rounds.
# --------------------------------------------------------------------------------------------

PHILOX_M = (0xD2511F53, 0xCD9E8D57)
PHILOX_W = (0x9E3779B9, 0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32-10 of counters ctr (uint32 array [..., 4]) under key (k0, k1): uint32 [..., 4]."""
    ctr = np.asarray(ctr, dtype=np.uint64)
    c0, c1, c2, c3 = (ctr[..., i] for i in range(4))
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    m0, m1 = np.uint64(PHILOX_M[0]), np.uint64(PHILOX_M[1])
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(PHILOX_W[0])) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W[1])) & _MASK32
        p0, p1 = c0 * m0, c2 * m1  # exact: 32 x 32 bits fit in 64
        c0, c1, c2, c3 = (p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _MASK32, (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _MASK32
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def sr_bits(outer, kpad, layout, seed):
    """16 random bits per element of an [outer, kpad] operand: element (i, k) takes half k % 2
    (low half first) of word (k % 8) // 2 of Philox4x32-10 at counter (k // 8, i, layout, 0)
    under key (seed mod 2^32, seed // 2^32).  layout: 0 row layout, 1 column layout, 2 mean."""
    blocks = kpad // 8
    ctr = np.zeros((outer, blocks, 4), np.uint64)
    ctr[..., 0] = np.arange(blocks, dtype=np.uint64)[None, :]
    ctr[..., 1] = np.arange(outer, dtype=np.uint64)[:, None]
    ctr[..., 2] = layout
    w = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))  # [outer, blocks, 4]
    halves = np.stack([w & 0xFFFF, w >> 16], axis=-1)                       # [outer, blocks, 4, 2]
    return halves.reshape(outer, kpad).astype(np.uint32)


def e2m1_encode_sr(v, u16):
    """E2M1 with stochastic rounding: the magnitude a = |v| lies between neighbouring grid values
    lo <= a < hi of {0, .5, 1, 1.5, 2, 3, 4, 6} and rounds to hi when u16 / 2^16 < (a - lo) /
    (hi - lo), else to lo; a >= 6 gives 6.  (a - lo) is exact in fp32 (lo <= a < 2 lo, or lo = 0)
    and hi - lo is a power of two, so the probability is exact.  The sign bit is v's."""
    v = np.asarray(v, dtype=F32)
    a = np.abs(v)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=F32)
    lo_i = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 6)
    lo, hi = grid[lo_i], grid[lo_i + 1]
    p = ((a - lo).astype(F32) / (hi - lo)).astype(F32)
    up = np.asarray(u16, np.float64) / 65536.0 < p
    c = np.where(a >= F32(6.0), 7, lo_i + up).astype(np.uint8)
    return c | (np.signbit(v).astype(np.uint8) << 3)


# --------------------------------------------------------------------------------------------
# Split.  [rainbus] 方法步骤详情: mu_X = (1/l) 1^T X over the l = b*s token rows and
# X_R = X - 1 mu_X; [paperlayer] §3 Method: the mean matrix is broadcast, never materialized.
# --------------------------------------------------------------------------------------------

def column_mean(x):
    """Column mean over the token rows: (mu in fp64, mu rounded once to fp32).

    Sums are taken in fp64 over the (bf16 or fp32) input values.  l == 0 gives zeros.
    """
    x = np.asarray(x, dtype=np.float64)
    l = x.shape[0]
    if l == 0:
        z = np.zeros(x.shape[1])
        return z, z.astype(F32)
    mu64 = np.sum(x, axis=0) / l
    return mu64, mu64.astype(F32)


def residual(x, mu32):
    """r_ij = fl32(x_ij - mu_j): one fp32 subtraction per element."""
    return np.asarray(x, dtype=F32) - np.asarray(mu32, dtype=F32)[None, :]


# --------------------------------------------------------------------------------------------
# Optional 16x16 Hadamard.  [rainbus] 前置知识 / Hadamard变换: reshape to [l, m/16, 16] and
# rotate the last dimension with a 16x16 Hadamard; 技术新颖性: Averis and Hadamard combine
# (split first, then smooth).  Reading: Sylvester order, scaled by 1/4 so it is orthogonal.
# --------------------------------------------------------------------------------------------

def hadamard16_f32(r):
    """Rotate each 16-element block along the last axis by H16/4 using fp32 butterflies.

    Stages h = 1, 2, 4, 8 in that order; each pairs elements j and j+h (bit h of j clear)
    into (a + b, a - b).  The final multiply by 0.25 is exact.
    """
    r = np.asarray(r, dtype=F32)
    shp = r.shape
    assert shp[-1] % 16 == 0
    v = r.reshape(-1, 16)
    for h in (1, 2, 4, 8):
        v = v.reshape(-1, 16 // (2 * h), 2, h)
        a = v[:, :, 0, :]
        b = v[:, :, 1, :]
        v = np.stack([a + b, a - b], axis=2).reshape(-1, 16)
    return (v * F32(0.25)).reshape(shp)


def sylvester16():
    """H16 built by the Sylvester recursion H_2k = [[H_k, H_k], [H_k, -H_k]]."""
    h = np.ones((1, 1))
    while h.shape[0] < 16:
        h = np.block([[h, h], [h, -h]])
    return h


def unrotate16_f64(v):
    """Exact (fp64) inverse of the /4-scaled Sylvester rotation along the last axis."""
    v = np.asarray(v, dtype=np.float64)
    shp = v.shape
    return (v.reshape(-1, 16) @ (sylvester16() / 4.0)).reshape(shp)


# --------------------------------------------------------------------------------------------
# Blockwise quantizer Q_b.  [rainbus] 块量化 and 方法步骤详情 (Q_b applied independently to the
# mean, the residual and W); [chatpaper] v1 abstract (standard quantization kernels).
# --------------------------------------------------------------------------------------------

class QTensor:
    """Packed result of Q_b on an [outer, k_pad] operand, blocks along the last axis.

    codes:  uint8 [outer, k_pad/2], element 2i in bits 3:0 and 2i+1 in bits 7:4.
    scales: uint8 [outer, k_pad/g]; E4M3 codes (NVFP4) or E8M0 codes = E + 127 (MXFP4).
    s_dec:  fp32 tensor decode scale (NVFP4) or None.
    k:      logical length along K (before padding).  rotated: Hadamard applied along K.
    """

    def __init__(self, codes, scales, s_dec, fmt, k, rotated):
        self.codes, self.scales, self.s_dec = codes, scales, s_dec
        self.fmt, self.k, self.rotated = fmt, k, rotated

    @property
    def outer(self):
        return self.codes.shape[0]

    @property
    def k_pad(self):
        return self.codes.shape[1] * 2


def pack_nibbles(c):
    c = np.asarray(c, dtype=np.uint8)
    return (c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)


def unpack_nibbles(b):
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def nvfp4_tensor_scale(amax):
    """s_dec = fl32(amax / 2688); 2688 = 6 * 448 maps the tensor max onto E2M1 max x E4M3 max."""
    return F32(F32(amax) / F32(2688.0))


def quantize_nvfp4(r, s_dec, u16=None):
    """NVFP4-style Q_b along the last axis of fp32 r [outer, K], K % 16 == 0.

    Per 16-block b with a_b = max |r|:
      e_b = E4M3(fl(fl(a_b / 6) / s_dec)); S_b = fl(val(e_b) * s_dec); R_b = fl(1 / S_b);
      codes = E2M1(fl(r * R_b)).
    Blocks with s_dec == 0, e_b == 0 or S_b below 2^-126 get all-zero codes.  u16 (uint [outer, K]):
    stochastic rounding with these random bits instead of round to nearest.
    """
    r = np.asarray(r, dtype=F32)
    outer, K = r.shape
    blk = r.reshape(outer, K // 16, 16)
    amax = np.max(np.abs(blk), axis=2) if K else np.zeros((outer, 0), F32)
    s_dec = F32(s_dec)
    if s_dec == 0:
        return np.zeros((outer, K // 2), np.uint8), np.zeros((outer, K // 16), np.uint8)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        t = (amax / F32(6.0)).astype(F32)
        t = (t / s_dec).astype(F32)
        e = e4m3_encode(t)
        S = (e4m3_value(e).astype(F32) * s_dec).astype(F32)
        R = (F32(1.0) / S).astype(F32)
        v = (blk * R[:, :, None]).astype(F32)
        codes = e2m1_encode(v) if u16 is None else e2m1_encode_sr(v, u16.reshape(outer, K // 16, 16))
    dead = (e == 0) | (S < F32(2.0 ** -126))
    codes[dead] = 0
    return pack_nibbles(codes.reshape(outer, K)), e


def quantize_mxfp4(r, u16=None):
    """MXFP4 Q_b along the last axis of fp32 r [outer, K], K % 32 == 0.

    Per 32-block: E = mx_scale_exponent(a_b); codes = E2M1(r * 2^-E) (exact scaling);
    scale byte = E + 127.  All-zero blocks get all-zero codes.  u16: stochastic rounding bits.
    """
    r = np.asarray(r, dtype=F32)
    outer, K = r.shape
    blk = r.reshape(outer, K // 32, 32)
    amax = np.max(np.abs(blk), axis=2) if K else np.zeros((outer, 0), F32)
    E = mx_scale_exponent(amax)
    R = np.ldexp(np.ones(E.shape, F32), -E).astype(F32)
    v = (blk * R[:, :, None]).astype(F32)
    codes = e2m1_encode(v) if u16 is None else e2m1_encode_sr(v, u16.reshape(outer, K // 32, 32))
    codes[amax == 0] = 0
    return pack_nibbles(codes.reshape(outer, K)), (E + 127).astype(np.uint8)


def quantize(r, fmt, rotate=False, k=None, u16=None):
    """Q_b of the fp32 operand r [outer, K] along K; optional H16 first.  NVFP4 takes its
    tensor scale from this operand's own amax (after rotation).  u16: stochastic rounding."""
    r = np.asarray(r, dtype=F32)
    if rotate:
        r = hadamard16_f32(r)
    k = r.shape[1] if k is None else k
    if fmt == NVFP4:
        amax = F32(np.max(np.abs(r))) if r.size else F32(0)
        s_dec = nvfp4_tensor_scale(amax)
        codes, scales = quantize_nvfp4(r, s_dec, u16)
        return QTensor(codes, scales, s_dec, fmt, k, rotate)
    if fmt == MXFP4:
        codes, scales = quantize_mxfp4(r, u16)
        return QTensor(codes, scales, None, fmt, k, rotate)
    raise ValueError(fmt)


def dequantize(q):
    """DQ in fp64 (exact): e2m1(code) * val(e_b) * s_dec, or e2m1(code) * 2^E."""
    c = e2m1_value(unpack_nibbles(q.codes))
    g = BLOCK[q.fmt]
    if q.fmt == NVFP4:
        s = e4m3_value(q.scales) * np.float64(q.s_dec)
    else:
        s = np.ldexp(1.0, q.scales.astype(np.int64) - 127)
    return c * np.repeat(s, g, axis=1)


# --------------------------------------------------------------------------------------------
# Split + quantize of one tensor: activations X [l, m] or output gradients D [l, n]
# ([rainbus] 方法步骤详情, forward and backward stages), or W with the split off.
# --------------------------------------------------------------------------------------------

def round_up(a, b):
    return (a + b - 1) // b * b


def pad_k(r):
    """Zero-pad the last axis of an fp32 operand to a multiple of KPAD."""
    r = np.asarray(r, dtype=F32)
    out = np.zeros((r.shape[0], round_up(r.shape[1], KPAD)), dtype=F32)
    out[:, :r.shape[1]] = r
    return out


def split_quant(x, fmt, split=True, hadamard=False, mean=None, sr_seed=None):
    """Returns dict(mu64, mu32, row=QTensor [rows, cols], col=QTensor [cols, rows],
    mean=QTensor [1, cols] or None), each stored zero-padded along K to a multiple of KPAD.

    `mean` (fp32 [cols]) replaces the computed mean -- used to quantize with the exact mean
    vector another implementation produced.  split=False is the vanilla quantizer (also the
    one for weights): no mean, no mean operand.  sr_seed (uint64): E2M1 with stochastic
    rounding, random bits sr_bits(.., layout 0 / 1 / 2, seed) for the row / column / mean
    operand.
    """
    x = np.asarray(x)
    rows, cols = x.shape
    mu64 = None
    if split:
        if mean is None:
            mu64, mu32 = column_mean(x)
        else:
            mu32 = np.asarray(mean, dtype=F32)
        r = residual(x, mu32)
    else:
        mu32 = None
        r = np.asarray(x, dtype=F32)
    rp, cp = round_up(rows, KPAD), round_up(cols, KPAD)
    bits = (lambda o, kp, lay: None) if sr_seed is None else (lambda o, kp, lay: sr_bits(o, kp, lay, sr_seed))
    q_row = quantize(pad_k(r), fmt, rotate=hadamard, k=cols, u16=bits(rows, cp, 0))
    q_col = quantize(pad_k(r.T), fmt, rotate=hadamard, k=rows, u16=bits(cols, rp, 1))
    q_mean = quantize(pad_k(mu32[None, :]), fmt, rotate=hadamard, k=cols, u16=bits(1, cp, 2)) if split else None
    return dict(mu64=mu64, mu32=mu32, row=q_row, col=q_col, mean=q_mean)


# --------------------------------------------------------------------------------------------
# The three GEMMs with the mean terms.  [rainbus] 方法步骤详情:
#   Y     = 1_l (mu_X W) + X_R W
#   dL/dX = 1_l (mu_D W^T) + D_R W^T
#   dL/dW = X_R^T D_R + l mu_X^T mu_D  (cross terms vanish for zero-mean residuals)
# The *_dense functions take dequantized (or unquantized) fp64 operands, K-inner:
#   a [M, K], b [N, K]  ->  a @ b.T ; mean rows [K].
# --------------------------------------------------------------------------------------------

def fwd_dense(xr, mu, w_nk):
    """Y [l, n] = 1 (mu W) + X_R W with W given as [n, m] (K = m inner)."""
    y = np.asarray(xr, np.float64) @ np.asarray(w_nk, np.float64).T
    if mu is not None:
        y = y + (np.asarray(mu, np.float64) @ np.asarray(w_nk, np.float64).T)[None, :]
    return y


def dx_dense(dr, mu_d, w_mn):
    """dX [l, m] = 1 (mu_D W^T) + D_R W^T with W given as [m, n] (K = n inner)."""
    return fwd_dense(dr, mu_d, w_mn)


def dw_dense(xr_t, dr_t, mu_x, mu_d, l):
    """dW [m, n] = X_R^T D_R + l mu_X^T mu_D with X_R^T [m, L], D_R^T [n, L] (K = tokens)."""
    dw = np.asarray(xr_t, np.float64) @ np.asarray(dr_t, np.float64).T
    if mu_x is not None:
        dw = dw + float(l) * np.outer(np.asarray(mu_x, np.float64), np.asarray(mu_d, np.float64))
    return dw


def _mean_row(qm):
    """Dequantized mean for the weight-gradient rank-one term (rotation undone exactly)."""
    v = dequantize(qm)[0]
    return (unrotate16_f64(v) if qm.rotated else v)[:qm.k]


def linear_fwd(q_xr, q_mu, q_w):
    """Quantized forward GEMM: q_xr [l, m], q_mu [1, m] or None (vanilla), q_w [n, m]."""
    mu = dequantize(q_mu)[0, :q_mu.k] if q_mu is not None else None
    return fwd_dense(dequantize(q_xr)[:, :q_xr.k], mu, dequantize(q_w)[:, :q_w.k])


def linear_bwd_dx(q_dr, q_mu, q_w):
    """Quantized input-gradient GEMM: q_dr [l, n], q_mu [1, n] or None, q_w [m, n]."""
    return linear_fwd(q_dr, q_mu, q_w)


def linear_bwd_dw(q_xr_t, q_dr_t, q_mu_x, q_mu_d, l):
    """Quantized weight-gradient GEMM: q_xr_t [m, L_pad], q_dr_t [n, L_pad] (K = tokens)."""
    mx = _mean_row(q_mu_x) if q_mu_x is not None else None
    md = _mean_row(q_mu_d) if q_mu_d is not None else None
    return dw_dense(dequantize(q_xr_t), dequantize(q_dr_t), mx, md, l)


# --------------------------------------------------------------------------------------------
# Grouped (MoE) variant: every step above applied per expert to its own contiguous token
# slice [offsets[e], offsets[e+1]).  [rainbus] 实验结果 (the 7B-A1.5B MoE is trained with
# Averis); the per-expert split on each expert's slice is the plain reading.
# --------------------------------------------------------------------------------------------

def split_quant_grouped(x, offsets, fmt, split=True, hadamard=False, means=None):
    out = []
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        mean = None if means is None else means[e]
        out.append(split_quant(x[a:b], fmt, split=split, hadamard=hadamard, mean=mean)
                   if b > a else None)
    return out


def linear_fwd_grouped(sq_x, q_ws, offsets, n):
    """Stack of per-expert forward outputs, [total_tokens, n]; empty experts contribute nothing."""
    ys = []
    for e, s in enumerate(sq_x):
        if s is None:
            continue
        ys.append(linear_fwd(s["row"], s["mean"], q_ws[e]))
    return np.concatenate(ys, axis=0) if ys else np.zeros((0, n))


def linear_bwd_dx_grouped(sq_d, q_ws, offsets, m):
    """Stack of per-expert input gradients, [total_tokens, m]; q_ws[e] is expert e's K = n weight."""
    ds = []
    for e, s in enumerate(sq_d):
        if s is None:
            continue
        ds.append(linear_bwd_dx(s["row"], s["mean"], q_ws[e]))
    return np.concatenate(ds, axis=0) if ds else np.zeros((0, m))


def linear_bwd_dw_grouped(sq_x, sq_d, offsets, m, n):
    """Per-expert dW [E, m, n]; an empty expert's dW is zero."""
    E = len(offsets) - 1
    out = np.zeros((E, m, n))
    for e in range(E):
        if sq_x[e] is None:
            continue
        l_e = int(offsets[e + 1] - offsets[e])
        out[e] = linear_bwd_dw(sq_x[e]["col"], sq_d[e]["col"], sq_x[e]["mean"],
                               sq_d[e]["mean"], l_e)
    return out


# --------------------------------------------------------------------------------------------
# Producers of a transformer block's linear inputs, whose column statistics the split can take
# instead of reading X again.  The pages name the model (Qwen3: RMSNorm, SwiGLU) but not these
# operations' arithmetic; the definitions are the published ones, in fp32 with one rounding per
# operation as the kernels do them, the output rounded to bf16.  Only the sum of squares is
# taken in fp64 here (the kernels sum in fp32), and exp is the correctly rounded one.
# --------------------------------------------------------------------------------------------

def round_bf16(v):
    """fp32 -> bf16 (round to nearest even, finite values), returned as fp32."""
    u = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def rmsnorm(x, w, eps, out_bf16=True):
    """RMSNorm (Zhang and Sennrich, 2019): y = x * (1 / sqrt(mean_c(x^2) + eps)) * w per row.
    fp32 steps: ms = fl(fl(s) * fl(1 / cols)), rs = fl(1 / fl(sqrt(fl(ms + eps)))),
    y = fl(fl(x * rs) * w), with s the fp64 sum of squares rounded to fp32."""
    x = np.asarray(x, np.float32)
    cols = x.shape[1]
    s = np.float32((x.astype(np.float64) ** 2).sum(axis=1)) if x.size else np.zeros(x.shape[0], np.float32)
    ms = np.float32(s) * np.float32(np.float32(1.0) / np.float32(cols))
    rs = np.float32(1.0) / np.sqrt(np.float32(ms + np.float32(eps)), dtype=np.float32)
    y = (x * rs[:, None]) * np.asarray(w, np.float32)[None, :]
    return round_bf16(y) if out_bf16 else y.astype(np.float32)


def swiglu(g, u, out_bf16=True):
    """SwiGLU gate (Shazeer, 2020): y = silu(g) * u, silu(g) = g / (1 + exp(-g)); fp32 steps,
    exp correctly rounded to fp32."""
    g = np.asarray(g, np.float32)
    e = np.float32(np.exp(-g.astype(np.float64)))
    y = (g / (np.float32(1.0) + e)) * np.asarray(u, np.float32)
    return round_bf16(y) if out_bf16 else y.astype(np.float32)


# --------------------------------------------------------------------------------------------
# Error statistic used for the pages' directional claim ([paperlayer] D Output-Gradient Mean
# Centering: centering lowers the relative NVFP4 quantization error).
# --------------------------------------------------------------------------------------------

def relative_error(approx, exact):
    exact = np.asarray(exact, np.float64)
    return float(np.linalg.norm(np.asarray(approx, np.float64) - exact) / np.linalg.norm(exact))


def reconstruct(sq, rows):
    """X ~ DQ(Q(X_R)) + 1 DQ(Q(mu)) from the row layout (unrotated operands only)."""
    xr = dequantize(sq["row"])[:, :sq["row"].k]
    if sq["mean"] is not None:
        xr = xr + dequantize(sq["mean"])[:, :sq["mean"].k]
    return xr[:rows]

