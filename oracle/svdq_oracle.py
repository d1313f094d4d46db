"""Plain, slow, obviously-correct CPU oracle (numpy) for the SVDQuant linear layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. It shares no code, table or helper with the GPU library.

What it computes (sources are the pages this project follows):

* The SVDQuant overview figure of the Nunchaku README ("Method > Quantization method - SVDQuant",
  stages 1-3): outliers are migrated from the activations into the weights by a per-channel
  smoothing (X_hat = X diag(lambda)^-1, W_hat = diag(lambda) W); W_hat is split by a truncated SVD
  into a low-rank part L1 L2 kept in 16 bits and a residual R = W_hat - L1 L2 that is quantized
  to 4 bits together with X_hat. The layer is therefore

      Y = X_hat L1 L2 + dequant(Q4(X_hat) Q4(R)) + b.

* The engine-design figure of the same README ("Nunchaku engine design", panels (a) and (b)):
  the down projection X_hat L1 shares its input with the activation quantizer and the up
  projection shares its output with the 4-bit product. Fusion changes no value, so the oracle
  computes each piece separately.

* The Diffusers blog on Nunchaku Lite ("From SVDQuant to Nunchaku Lite" and the
  ``quantization_config`` example): ``svdq_w4a4`` layers with a rank-32 low-rank branch for
  attention/MLP, ``awq_w4a16`` layers (int4 weights, group 64, 16-bit activations) for the
  modulation / adaptive-norm projections, compute dtype bfloat16.

Readings where the pages are silent (each is a documented choice, applied identically here and
on the GPU): symmetric INT4 with one float32 scale per group of 64 consecutive inputs along K;
scale = float32(absmax) / float32(7) with IEEE division; code = clamp(round_half_even(x / scale),
-8, 7) with an IEEE float32 division; a group whose computed scale is 0 gets scale 0 and codes 0;
X_hat = float32(x) * float32(1/lambda) (one float32 multiply); the down projection consumes
bf16(X_hat) and its result T is stored as bf16; the output is rounded to bf16. The W4A16 scale
is bf16(float32(absmax)/7) and its codes are computed against that rounded scale.
The main product is evaluated in float64 (the exact integer group sums times the float32
scales), the smoothing/SVD preparation in float64.

* The same Diffusers blog ("From SVDQuant to Nunchaku Lite") names a dedicated GELU/MLP execution
  path of the Nunchaku engine. The pages give no formula; the reading here is the tanh form of
  GELU used by FLUX-style MLPs, applied to the layer's unrounded output before the bf16 rounding:
  Y = bf16( gelu_tanh(Y_pre) ), gelu_tanh(v) = v/2 (1 + tanh( sqrt(2/pi) (v + 0.044715 v^3) )).

* The same blog's section on structural rewrites: FLUX's attention projects Q, K and V, splits
  heads, RMS-normalises Q and K per head (norm_q, norm_k) and applies the rotary embedding; the
  engine fuses the three projections into one to_qkv (Q, K, V concatenated in that order along the
  output dimension) followed by a fused norm + rotary operator. Readings: head dimension 128, one
  RMS weight vector per Q and K shared by all heads, eps = 1e-6, the normalisation applied to the
  projection's bf16 output (what an unfused pipeline reads), the rotary embedding on interleaved
  pairs (2i, 2i+1) with per-token cos/sin tables, one bf16 rounding at the end; V unchanged.
"""
from __future__ import annotations

import numpy as np

GROUP = 64  # INT4 group size along K (quantization_config of the Diffusers blog: group_size 64 for int4)
QMIN, QMAX = -8, 7

__all__ = [
    "GROUP", "bf16_round", "smoothing_factors", "svdq_decompose", "int4_quantize_rows",
    "quantize_weights_w4a4", "smooth_activations", "quantize_activations", "lowrank_down",
    "group_sums", "dequant_product", "svdq_linear", "svdq_layer", "quantize_weights_w4a16",
    "awq_linear", "gelu_tanh", "svdq_linear_gelu", "qkv_norm_rope",
    "svdq_layer_naive", "MX_BLOCK", "E2M1_VALUES", "e2m1_decode", "e2m1_round", "mxfp4_quantize_rows", "mxfp4_dequant",
    "quantize_activations_mxfp4", "quantize_weights_mxfp4", "svdq_linear_mxfp4", "svdq_layer_mxfp4",
]


# ----------------------------------------------------------------------------------------------
# 16-bit storage
# ----------------------------------------------------------------------------------------------
def bf16_round(a) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 values.

    Works on the float32 bit pattern: add 0x7FFF plus the lowest kept bit, then clear the low
    16 bits. Inputs are finite (non-finite values are outside this oracle's domain).
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).reshape(f.shape)


# ----------------------------------------------------------------------------------------------
# Offline preparation (overview figure, stages 2 and 3)
# ----------------------------------------------------------------------------------------------
def smoothing_factors(x: np.ndarray, w: np.ndarray):
    """Per-input-channel smoothing (stage 2 of the SVDQuant overview figure).

    lambda_k = sqrt(max_m |x[m,k]| / max_n |w[k,n]|) in float64 (the migration-strength-1/2 rule of
    SmoothQuant, which the README lists as the related work this stage builds on); lambda_k = 1
    when either maximum is 0. The runtime carries inv_k = float32(1/lambda_k) and the weights are
    scaled by lambda'_k = 1/float64(inv_k), so that X diag(inv) diag(lambda') W = X W exactly in
    real arithmetic.
    Returns (inv float32 [K], lam_prime float64 [K]).
    """
    xmax = np.max(np.abs(x.astype(np.float64)), axis=0)
    wmax = np.max(np.abs(w.astype(np.float64)), axis=1)
    lam = np.ones(x.shape[1], dtype=np.float64)
    ok = (xmax > 0) & (wmax > 0)
    lam[ok] = np.sqrt(xmax[ok] / wmax[ok])
    inv = (1.0 / lam).astype(np.float32)
    lam_prime = 1.0 / inv.astype(np.float64)
    return inv, lam_prime


def svdq_decompose(x: np.ndarray, w: np.ndarray, rank: int, svd=None):
    """Smoothing + truncated SVD + residual (stages 2-3 of the SVDQuant overview figure).

    x: float32 [M, K] activations used for calibration; w: float32 [K, N] weights (x @ w).
    W_hat = diag(lambda') w; W_hat = U S V^T; L1 = U_r S_r, L2 = V_r^T (float64).
    The runtime factors are bf16(L1), bf16(L2); the residual that gets quantized is
    R = W_hat - bf16(L1) bf16(L2), computed in float64 and stored as float32.
    ``svd`` may pass in numpy.linalg.svd(W_hat, full_matrices=False) of this same W_hat, so that
    several ranks of one layer share one factorisation.
    """
    inv, lam_prime = smoothing_factors(x, w)
    w_hat = lam_prime[:, None] * w.astype(np.float64)
    u, s, vt = np.linalg.svd(w_hat, full_matrices=False) if svd is None else svd
    l1 = u[:, :rank] * s[:rank]
    l2 = vt[:rank, :]
    l1_b = bf16_round(l1.astype(np.float32))
    l2_b = bf16_round(l2.astype(np.float32))
    resid = (w_hat - l1_b.astype(np.float64) @ l2_b.astype(np.float64)).astype(np.float32)
    return {"inv": inv, "lam_prime": lam_prime, "w_hat": w_hat, "sigma": s, "l1": l1, "l2": l2,
            "l1_bf16": l1_b, "l2_bf16": l2_b, "resid": resid}


# ----------------------------------------------------------------------------------------------
# Symmetric INT4, one float32 scale per group of 64 along the reduction axis
# ----------------------------------------------------------------------------------------------
def int4_quantize_rows(v: np.ndarray):
    """Quantize each row of float32 ``v`` [rows, K] in groups of 64 consecutive entries.

    scale = float32(absmax) / float32(7) (IEEE); code = clamp(rint_even(v / scale), -8, 7) with
    an IEEE float32 division; a group whose scale is 0 gets codes 0.
    Returns (codes int8 [rows, K], scales float32 [rows, K/64]).
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    rows, K = v.shape
    assert K % GROUP == 0
    G = K // GROUP
    vg = v.reshape(rows, G, GROUP)
    amax = np.max(np.abs(vg), axis=2)                               # exact
    scale = (amax / np.float32(7.0)).astype(np.float32)             # float32 / float32: IEEE
    codes = np.zeros((rows, G, GROUP), dtype=np.int8)
    nz = scale != 0
    with np.errstate(divide="ignore", invalid="ignore"):
        q = vg / scale[:, :, None]                                  # float32 division
    q = np.clip(np.rint(q), QMIN, QMAX)                             # round half to even, clamp
    codes[nz] = q[nz].astype(np.int8)
    return codes.reshape(rows, K), scale


def quantize_weights_w4a4(resid: np.ndarray):
    """Q4 of the residual R [K, N] along K, per output column.

    Returns (codes int8 [K, N], scales float32 [K/64, N]).
    """
    c, s = int4_quantize_rows(np.ascontiguousarray(resid.T))
    return np.ascontiguousarray(c.T), np.ascontiguousarray(s.T)


def smooth_activations(x: np.ndarray, inv: np.ndarray) -> np.ndarray:
    """X_hat = float32(x) * inv (one float32 multiply per element, round to nearest even)."""
    return (x.astype(np.float32) * inv.astype(np.float32)[None, :]).astype(np.float32)


def lowrank_down(x_hat: np.ndarray, l1_bf16: np.ndarray) -> np.ndarray:
    """T = bf16( bf16(X_hat) @ bf16(L1) ): the 16-bit down projection (engine figure (a)/(b))."""
    xh16 = bf16_round(x_hat).astype(np.float64)
    return bf16_round((xh16 @ l1_bf16.astype(np.float64)).astype(np.float32))


def quantize_activations(x: np.ndarray, inv: np.ndarray, l1_bf16=None):
    """What the fused activation step produces: (codes int8 [M,K], scales float32 [K/64, M], T or None).

    Codes/scales: Q4 of X_hat per token along K. T: the rank-r down projection of X_hat.
    """
    xh = smooth_activations(x, inv)
    codes, sc = int4_quantize_rows(xh)
    t = None if l1_bf16 is None or l1_bf16.shape[1] == 0 else lowrank_down(xh, l1_bf16)
    return codes, np.ascontiguousarray(sc.T), t


# ----------------------------------------------------------------------------------------------
# The W4A4 product and the layer
# ----------------------------------------------------------------------------------------------
def group_sums(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """P[g, m, n] = sum_{k in group g} qa[m, k] * qw[k, n], exact integers (int64)."""
    M, K = qa.shape
    G = K // GROUP
    a = qa.astype(np.int64).reshape(M, G, GROUP)
    b = qw.astype(np.int64).reshape(G, GROUP, -1)
    return np.stack([a[:, g, :] @ b[g] for g in range(G)], axis=0)


def dequant_product(qa, sa, qw, sw) -> np.ndarray:
    """dequant(Q4(X_hat) Q4(R)) = (qa * sa) @ (qw * sw) in float64.

    qa int8 [M,K], sa float32 [K/64, M], qw int8 [K,N], sw float32 [K/64, N].
    """
    a = qa.astype(np.float64) * np.repeat(sa.T.astype(np.float64), GROUP, axis=1)
    b = qw.astype(np.float64) * np.repeat(sw.astype(np.float64), GROUP, axis=0)
    return a @ b


def svdq_linear(qa, sa, qw, sw, t=None, l2_bf16=None, bias=None):
    """Y = dequant(Q4(X_hat) Q4(R)) + T L2 + b, returned as (float64, bf16-rounded float32)."""
    y = dequant_product(qa, sa, qw, sw)
    if t is not None and l2_bf16 is not None and l2_bf16.shape[0] > 0:
        y = y + t.astype(np.float64) @ l2_bf16.astype(np.float64)
    if bias is not None:
        y = y + bias.astype(np.float64)[None, :]
    return y, bf16_round(y.astype(np.float32))


def gelu_tanh(v) -> np.ndarray:
    """GELU in its tanh form, in float64: v/2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (v + 0.044715 * v ** 3)))


def svdq_linear_gelu(qa, sa, qw, sw, t=None, l2_bf16=None, bias=None):
    """The up projection of an MLP with its activation: Y = bf16( gelu_tanh(Y_pre) ), Y_pre the
    float64 layer output of svdq_linear. Returns (float64 gelu(Y_pre), bf16-rounded float32)."""
    y_pre, _ = svdq_linear(qa, sa, qw, sw, t, l2_bf16, bias)
    g = gelu_tanh(y_pre)
    return g, bf16_round(g.astype(np.float32))


def qkv_norm_rope(y_bf16, heads, q_w, k_w, cos, sin, head_dim=128, eps=1e-6):
    """Per-head RMS normalisation and rotary embedding of the Q and K parts of a fused QKV output.

    y_bf16 float32 [M, 3 * heads * head_dim] holding the projection's bf16 values (Q | K | V);
    q_w, k_w [head_dim]; cos, sin [M, head_dim / 2] (the angle of pair i of token m). For Q and
    K, per token and head: u = v / sqrt(mean(v^2) + eps) * w, then pair (u[2i], u[2i+1]) ->
    (u[2i] c - u[2i+1] s, u[2i] s + u[2i+1] c) with c = cos[m, i], s = sin[m, i]; evaluated in
    float64 and rounded to bf16 once. V is returned unchanged. Returns float32 holding bf16."""
    y = np.asarray(y_bf16, dtype=np.float64)
    M, N = y.shape
    assert N == 3 * heads * head_dim
    out = y.copy()
    c = np.asarray(cos, dtype=np.float64)[:, None, :]
    s = np.asarray(sin, dtype=np.float64)[:, None, :]
    for part, w in ((0, q_w), (1, k_w)):
        v = y[:, part * heads * head_dim:(part + 1) * heads * head_dim].reshape(M, heads, head_dim)
        rms = np.sqrt(np.mean(v * v, axis=2, keepdims=True) + eps)
        u = v / rms * np.asarray(w, dtype=np.float64)[None, None, :]
        a, b = u[:, :, 0::2], u[:, :, 1::2]
        r = np.empty_like(u)
        r[:, :, 0::2] = a * c - b * s
        r[:, :, 1::2] = a * s + b * c
        out[:, part * heads * head_dim:(part + 1) * heads * head_dim] = r.reshape(M, heads * head_dim)
    res = bf16_round(out.astype(np.float32))
    res[:, 2 * heads * head_dim:] = np.asarray(y_bf16, dtype=np.float32)[:, 2 * heads * head_dim:]
    return res


def svdq_layer(x, inv, l1_bf16, l2_bf16, resid, bias=None):
    """The whole layer from its prepared inputs; returns a dict of every intermediate."""
    qa, sa, t = quantize_activations(x, inv, l1_bf16)
    qw, sw = quantize_weights_w4a4(resid)
    y64, y = svdq_linear(qa, sa, qw, sw, t, l2_bf16, bias)
    return {"qa": qa, "sa": sa, "t": t, "qw": qw, "sw": sw, "y64": y64, "y": y}


def svdq_layer_naive(x, inv, l1_bf16, l2_bf16, resid, bias=None):
    """The layer run the unfused way of the engine-design figure's panel (a): the 4-bit branch writes
    its 16-bit output Y0 = bf16(dequant(Q4(X_hat) Q4(R)) + b); a separate 16-bit down projection
    reads X again, T = bf16(X @ bf16(diag(inv) L1)) (the smoothing folded into L1, since it no longer
    passes through the quantizer); a separate up projection reads and rewrites the 16-bit output,
    Y = bf16(Y0 + T L2). The same quantities as svdq_layer with the two extra 16-bit roundings of
    that form. Returns the dict of svdq_layer with "y0", "l1s", "t" and "y" of the naive form."""
    qa, sa, _ = quantize_activations(x, inv, None)
    qw, sw = quantize_weights_w4a4(resid)
    y0 = dequant_product(qa, sa, qw, sw)
    if bias is not None:
        y0 = y0 + bias.astype(np.float64)[None, :]
    y0 = bf16_round(y0.astype(np.float32))
    l1s = bf16_round((inv.astype(np.float64)[:, None] * l1_bf16.astype(np.float64)).astype(np.float32))
    t = bf16_round((x.astype(np.float64) @ l1s.astype(np.float64)).astype(np.float32))
    y64 = y0.astype(np.float64) + t.astype(np.float64) @ l2_bf16.astype(np.float64)
    return {"qa": qa, "sa": sa, "qw": qw, "sw": sw, "y0": y0, "l1s": l1s, "t": t, "y64": y64,
            "y": bf16_round(y64.astype(np.float32))}


# ----------------------------------------------------------------------------------------------
# W4A16 (AWQ-style) projection: int4 weights, group 64, bf16 scales, 16-bit activations
# ----------------------------------------------------------------------------------------------
def quantize_weights_w4a16(w: np.ndarray):
    """int4 group-64 weights with bf16 scales: s = bf16(float32(absmax)/7); codes against s.

    w float32 [K, N]. Returns (codes int8 [K, N], scales float32 [K/64, N] holding bf16 values).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    K, N = w.shape
    G = K // GROUP
    wg = w.reshape(G, GROUP, N)
    amax = np.max(np.abs(wg), axis=1)
    s = bf16_round((amax / np.float32(7.0)).astype(np.float32))
    with np.errstate(divide="ignore", invalid="ignore"):
        q = wg / s[:, None, :]
    q = np.clip(np.rint(q), QMIN, QMAX)
    codes = np.zeros((G, GROUP, N), dtype=np.int8)
    nz = np.broadcast_to((s != 0)[:, None, :], q.shape)
    codes[nz] = q[nz].astype(np.int8)
    return codes.reshape(K, N), s


def awq_linear(x, codes, scales, bias=None):
    """Y = x @ (codes * scales) + b in float64; returns (float64, bf16-rounded float32)."""
    wdq = codes.astype(np.float64) * np.repeat(scales.astype(np.float64), GROUP, axis=0)
    y = x.astype(np.float64) @ wdq
    if bias is not None:
        y = y + bias.astype(np.float64)[None, :]
    return y, bf16_round(y.astype(np.float32))



# ----------------------------------------------------------------------------------------------
# The 4-bit float variant: MXFP4 (E2M1 elements, one E8M0 power-of-two scale per block of 32)
# ----------------------------------------------------------------------------------------------
# The pages name a 4-bit float precision for svdq_w4a4 layers beside INT4 (the Nunchaku README's
# news and performance notes on NVFP4, the Diffusers blog's quantization_config with precision
# "nvfp4" and group_size 16, the Z-Image guide's "INT4 vs NVFP4" table) but do not define the
# format. Reading: on CDNA4 the matrix cores take the OCP Microscaling (MX) formats natively, so
# the variant built here is MXFP4 as that specification defines it:
#   * an element is FP4 E2M1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit; the magnitudes
#     are 0, 0.5 (exponent field 0: mantissa x 0.5), 1, 1.5, 2, 3, 4, 6 (2^(E-1) (1 + M/2));
#     its 4-bit code is (S << 3) | (E << 1) | M;
#   * each block of 32 consecutive values along K shares one E8M0 scale X = 2^e (byte e + 127),
#     e = floor(log2(absmax)) - 2 (2 = the largest E2M1 exponent), clamped to [-127, 127];
#     an all-zero block gets byte 0;
#   * element = v / X rounded to the nearest E2M1 value, ties to the even mantissa, magnitudes
#     above 6 saturate to 6; the sign bit is the sign bit of v.
# The layer is otherwise unchanged: Y = X_hat L1 L2 + dequant(MXFP4(X_hat) MXFP4(R)) + b.

MX_BLOCK = 32
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)   # magnitude of codes 0..7, by the definition


def e2m1_decode(codes) -> np.ndarray:
    """4-bit E2M1 codes -> float64 values, from the field definition (not a table lookup)."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag)


def e2m1_round(q) -> np.ndarray:
    """Nearest E2M1 magnitude code (0..7) of |q| (float64), ties to the even code, saturating at 6:
    every candidate's distance is compared, the closest wins, an exact tie goes to the code whose
    mantissa bit (the lowest bit) is 0."""
    a = np.abs(np.asarray(q, dtype=np.float64))
    grid = np.array(E2M1_VALUES)
    d = np.abs(a[..., None] - grid)                        # exact: a is a float, grid values are dyadic
    best = np.argmin(d, axis=-1)                           # first (lowest) code among equal distances
    dmin = np.take_along_axis(d, best[..., None], axis=-1)[..., 0]
    nxt = np.minimum(best + 1, 7)
    tie = (np.take_along_axis(d, nxt[..., None], axis=-1)[..., 0] == dmin) & (nxt != best)
    code = np.where(tie & (best % 2 == 1), nxt, best)     # a tie between codes c, c+1: keep the even one
    return np.where(a > 6.0, 7, code).astype(np.int64)


def mxfp4_quantize_rows(v: np.ndarray):
    """MXFP4 of each row of float32 ``v`` [rows, K], blocks of 32 consecutive entries.

    Returns (codes uint8 [rows, K] holding 4-bit E2M1 codes, scales uint8 [rows, K/32] holding E8M0
    bytes)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    rows, K = v.shape
    assert K % MX_BLOCK == 0
    vb = v.reshape(rows, K // MX_BLOCK, MX_BLOCK).astype(np.float64)
    amax = np.max(np.abs(vb), axis=2)
    _, ex = np.frexp(amax)                                 # amax = f 2^ex, f in [0.5, 1): floor(log2) = ex - 1
    e = np.clip(ex - 1 - 2, -127, 127)
    e = np.where(amax == 0, -127, e)
    q = np.ldexp(vb, -e[:, :, None])                       # v / X, exact in float64
    mag = e2m1_round(q)
    sign = np.signbit(vb).astype(np.int64)
    codes = (sign << 3) | mag
    return codes.reshape(rows, K).astype(np.uint8), (e + 127).astype(np.uint8)


def mxfp4_dequant(codes, scales) -> np.ndarray:
    """float64 values of MXFP4 rows: codes uint8 [rows, K], scales uint8 [rows, K/32]."""
    c = np.asarray(codes)
    rows, K = c.shape
    e = np.asarray(scales, dtype=np.int64) - 127
    return e2m1_decode(c) * np.ldexp(1.0, np.repeat(e, MX_BLOCK, axis=1))


def quantize_activations_mxfp4(x: np.ndarray, inv: np.ndarray, l1_bf16=None):
    """The fused activation step of the MXFP4 layer: (codes uint8 [M, K], E8M0 scales uint8
    [M, K/32], T or None); T exactly as in the INT4 layer."""
    xh = smooth_activations(x, inv)
    codes, sc = mxfp4_quantize_rows(xh)
    t = None if l1_bf16 is None or l1_bf16.shape[1] == 0 else lowrank_down(xh, l1_bf16)
    return codes, sc, t


def quantize_weights_mxfp4(resid: np.ndarray):
    """MXFP4 of the residual R [K, N] along K, per output column: (codes uint8 [N, K], scales
    uint8 [N, K/32]) (one row per output column)."""
    return mxfp4_quantize_rows(np.ascontiguousarray(resid.T))


def svdq_linear_mxfp4(qa, sa, qw, sw, t=None, l2_bf16=None, bias=None):
    """Y = dequant(MXFP4(X_hat)) dequant(MXFP4(R)) + T L2 + b in float64; returns (float64,
    bf16-rounded float32). qa/sa per token, qw/sw per output column."""
    y = mxfp4_dequant(qa, sa) @ mxfp4_dequant(qw, sw).T
    if t is not None and l2_bf16 is not None and l2_bf16.shape[0] > 0:
        y = y + t.astype(np.float64) @ l2_bf16.astype(np.float64)
    if bias is not None:
        y = y + bias.astype(np.float64)[None, :]
    return y, bf16_round(y.astype(np.float32))


def svdq_layer_mxfp4(x, inv, l1_bf16, l2_bf16, resid, bias=None):
    """The MXFP4 layer from its prepared inputs; returns a dict of every intermediate."""
    qa, sa, t = quantize_activations_mxfp4(x, inv, l1_bf16)
    qw, sw = quantize_weights_mxfp4(resid)
    y64, y = svdq_linear_mxfp4(qa, sa, qw, sw, t, l2_bf16, bias)
    return {"qa": qa, "sa": sa, "t": t, "qw": qw, "sw": sw, "y64": y64, "y": y}
