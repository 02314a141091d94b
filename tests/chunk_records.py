"""fp64 reference of the two-stage prefill's chunk records and their byte layout
(test infrastructure: the GPU tests compare stage 1's records with these, and
feed stage 2 records built here).

Chunkwise form of the recurrence ("Kimi 모델 분석", rlaope.github.io, section on
putting the recurrence on the GPU), for one 32-token chunk with decays a [32, d_k]
(tokens past the sequence end: a = 1, k = q = 0, beta = 0):
  pre_t = prod_{s<=t} a_s, suf_t = prod_{s>t} a_s, gamma = pre_31,
  KG = k pre, QG = q pre, KH = k suf,
  L_ij = beta_i sum_c k_ic k_jc r_c(i,j) (j < i), P_ij = sum_c q_ic k_jc r_c(i,j) (j <= i),
  r(i,j) = prod_{j<s<=i} a_s, T = (I + L)^{-1} diag(beta); the record holds the
  output's intra-chunk operator P T in place of P.
Record: fp16 fragments of 64 lanes x 8 values (lane 16 g + n, slot e) and gamma
(fp32), in the order KG, T, -KH^T, gamma, QG, -P T, its remainder:
  KG, QG [rt][kb]: token 16 rt + n, channel 32 kb + st(g, e); T, -P T [rt] (then
  its fp16 remainder, same layout): row
  16 rt + n, column st(g, e); -KH^T [i]: channel 16 i + n, token st(g, e);
  st(g, e) = 4 g + e (e < 4) or 16 + 4 g + e - 4.
"""
import numpy as np

CS = 32


def offsets(dk):
    """Byte offsets: the state part (KG, T, -KH^T, gamma), then the output part
    (QG, -P T, its remainder)."""
    nkb, nkt = dk // 32, dk // 16
    o = {"KG": 0}
    o["TT"] = o["KG"] + 2 * nkb * 1024
    o["KH"] = o["TT"] + 2 * 1024
    o["GAM"] = o["KH"] + nkt * 1024
    o["OUT"] = o["QG"] = o["GAM"] + dk * 4
    o["PP"] = o["QG"] + 2 * nkb * 1024
    o["PL"] = o["PP"] + 2 * 1024
    o["BYTES"] = o["PL"] + 2 * 1024
    return o


def _st(g, e):
    return 4 * g + e if e < 4 else 16 + 4 * g + (e - 4)


# index maps: for a fragment, (lane, slot) -> (row-in-block n, column st(g, e))
_LANE = np.arange(64)[:, None].repeat(8, 1)
_SLOT = np.arange(8)[None, :].repeat(64, 0)
_ROW = _LANE % 16
_COL = np.vectorize(_st)(_LANE // 16, _SLOT)


def chunk_operands(q, k, a, beta):
    """fp64 (KG, QG, KH, T, P, gamma) of one chunk; q, k, a: [32, d_k], beta: [32]."""
    q, k, a, beta = (np.asarray(x, np.float64) for x in (q, k, a, beta))
    pre = np.cumprod(a, axis=0)
    suf = np.ones_like(a)
    for t in range(CS - 2, -1, -1):
        suf[t] = suf[t + 1] * a[t + 1]
    L = np.zeros((CS, CS))
    P = np.zeros((CS, CS))
    for i in range(CS):
        r = np.ones(a.shape[1])
        for j in range(i, -1, -1):  # r = prod_{j<s<=i} a_s
            if j < i:
                r = r * a[j + 1]
                L[i, j] = beta[i] * np.sum(k[i] * k[j] * r)
            P[i, j] = np.sum(q[i] * k[j] * r)
    T = np.linalg.solve(np.eye(CS) + L, np.diag(beta))
    return k * pre, q * pre, k * suf, T, P, pre[-1]


def pack(dk, KG, QG, KH, T, P, gam):
    """The record bytes (uint8) of one chunk's operands (P: the chunk's P; the
    record stores -P T)."""
    o = offsets(dk)
    rec = np.zeros(o["BYTES"], np.uint8)
    h = rec.view(np.float16)

    def put(base, f, m):  # m: [64, 8] values of fragment f
        s = (base + f * 1024) // 2
        h[s:s + 512] = m.astype(np.float16).reshape(-1)

    for rt in range(2):
        for kb in range(dk // 32):
            put(o["KG"], rt * (dk // 32) + kb, KG[16 * rt + _ROW, 32 * kb + _COL])
            put(o["QG"], rt * (dk // 32) + kb, QG[16 * rt + _ROW, 32 * kb + _COL])
        put(o["TT"], rt, T[16 * rt + _ROW, _COL])
        npt = -(P @ T)[16 * rt + _ROW, _COL]
        put(o["PP"], rt, npt)
        put(o["PL"], rt, npt - npt.astype(np.float16).astype(np.float64))
    for i in range(dk // 16):
        put(o["KH"], i, -KH[_COL, 16 * i + _ROW])
    rec[o["GAM"]:o["OUT"]].view(np.float32)[:] = gam
    return rec


def unpack(dk, rec):
    """Inverse of pack: (KG, QG, KH, T, P T, gamma) as float64 from record bytes."""
    o = offsets(dk)
    h = rec.view(np.float16).astype(np.float64)

    def get(base, f):
        s = (base + f * 1024) // 2
        return h[s:s + 512].reshape(64, 8)

    KG, QG, KH = np.zeros((CS, dk)), np.zeros((CS, dk)), np.zeros((CS, dk))
    T, P = np.zeros((CS, CS)), np.zeros((CS, CS))
    for rt in range(2):
        for kb in range(dk // 32):
            KG[16 * rt + _ROW, 32 * kb + _COL] = get(o["KG"], rt * (dk // 32) + kb)
            QG[16 * rt + _ROW, 32 * kb + _COL] = get(o["QG"], rt * (dk // 32) + kb)
        T[16 * rt + _ROW, _COL] = get(o["TT"], rt)
        P[16 * rt + _ROW, _COL] = -(get(o["PP"], rt) + get(o["PL"], rt))
    for i in range(dk // 16):
        KH[_COL, 16 * i + _ROW] = -get(o["KH"], i)
    return KG, QG, KH, T, P, rec[o["GAM"]:o["OUT"]].view(np.float32).astype(np.float64)


def records(q, k, alpha, beta):
    """Records of every chunk of B sequences ([B,T,H,d] host arrays), in slot order
    (b * ceil(T/32) + c) * H + h, as one uint8 array."""
    q, k, alpha, beta = (np.asarray(x, np.float64) for x in (q, k, alpha, beta))
    B, T, H, dk = q.shape
    nc = (T + CS - 1) // CS
    out = []
    for b in range(B):
        for c in range(nc):
            for h in range(H):
                rows = min(CS, T - c * CS)
                qq, kk = np.zeros((CS, dk)), np.zeros((CS, dk))
                aa, bb = np.ones((CS, dk)), np.zeros(CS)
                sl = slice(c * CS, c * CS + rows)
                qq[:rows], kk[:rows], aa[:rows], bb[:rows] = q[b, sl, h], k[b, sl, h], alpha[b, sl, h], beta[b, sl, h]
                out.append(pack(dk, *chunk_operands(qq, kk, aa, bb)))
    return np.concatenate(out)
