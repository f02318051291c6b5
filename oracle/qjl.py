"""Plain fp64 CPU oracle of 1-bit QJL KV-cache compression and decode attention.

TEST INFRASTRUCTURE ONLY: see the package docstring for who may import it.

Every function follows a passage of the pages it cites and keeps the pages' order of steps. It is
written for a reader who checks it against the pages by eye: no blocking, no fusion, no reordering
beyond evaluating independent tokens in slices. Floating point is fp64 except where a float decides
an integer that the kernels also decide (the value codes), where the steps are spelled out in IEEE
float32 so both sides take the decision in the same precision.

Sources (page title, then section):
  [QJL]   "QJL: 1-Bit Quantized JL Transform for KV Cache Quantization with Zero Overhead"
          (AI-written summary on atlas.scime.ai) - "Approach", "Surprising findings", "Limitations".
  [1BIT]  "Your Brain Already Runs on 1-Bit Keys" (0x01.fyi blog) - "The 1-Bit Breakthrough",
          "But Wait. Don't the Small Dims Overpower?", "Why Truncation Kills".
  [2NUM]  "2 numbers out of 128 destroy the entire KV cache" (Towards AI) - "The Obvious Fix: Use
          Fewer Bits", "Small Errors, Exponential Damage", "Why Outliers Destroy Quantization".
  [HARD]  "Why Compressing the KV Cache Is Hard" (TurboQuant slides, section 5) - "Just Round
          Everything - The Naive Approach", "A Worked Example: When Rounding Ruins Attention".

Readings taken where the pages are silent:
  * estimator constant: score = sqrt(pi/2)/m * ||k|| * <S q, sign(S k)>; the pages only say the
    asymmetric estimator is unbiased [QJL "Approach"]; sqrt(pi/2) is what makes it unbiased for
    Gaussian S (E[<s,q> sign<s,k>] = sqrt(2/pi) <q,k>/||k||);
  * outlier copy [QJL "Approach"]: an independent JL matrix S_out applied to the outlier channels
    only; the same channel mask splits both key and query; the two estimates are added;
  * sign(0) is read as +1 (bit = 1 when the projection is >= 0);
  * bit order: bit i of uint32 word w holds projection 32 w + i; inlier words, then outlier words;
  * norms are stored as IEEE binary16, round-to-nearest-even ("16-bit norm", [1BIT]);
  * value quantization is per token and KV head over the whole head dimension, min/max range with
    2^b - 1 equal steps and round-to-nearest [2NUM "The Obvious Fix"]; min and step stored as fp16;
  * attention: z = sm_scale * score, softmax over all N keys (no mask), weighted sum of values;
  * outlier channels of a KV head [2NUM "The Real Problem: Outlier Channels", HARD "The Third
    Problem: Magnitude Outliers"]: the n_out channels with the largest mean magnitude |k_c| over all
    keys of that head seen so far (every sequence and token of the prefill), the lower channel first
    on equal means; returned in ascending channel order;
  * two-sided estimator [QJL "Surprising findings": signs on both sides estimate the cosine with a
    bias]: per part, ||q_part|| * ||k_part|| / m_part * <sign(S q_part), sign(S k_part)> (the mean
    sign agreement scaled by both norms, expectation ||q|| ||k|| (1 - 2 theta / pi)); the query
    signs take sign(0) = +1 like the keys; the parts add as for the one-sided estimator;
  * rotate-then-sign keys [1BIT "The 1-Bit Breakthrough", "But Wait. Don't the Small Dims
    Overpower?"]: an orthogonal rotation R (m = d), key reconstructed as norm x signs scaled to the
    key's norm, ||k|| sign(R k) / sqrt(d), dotted with the rotated query R q.
"""
from __future__ import annotations

import math

import numpy as np

SQRT_HALF_PI = math.sqrt(math.pi / 2.0)
_SLICE = 8192          # keys per slice when scoring (bounds memory only)


# ----------------------------------------------------------------------------- helpers

def fp16(x) -> np.ndarray:
    """IEEE binary16, round-to-nearest-even (numpy's correctly rounded conversion)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def outlier_mask(d: int, channels) -> np.ndarray:
    """1.0 on the outlier channels of one KV head, 0.0 elsewhere (length d)."""
    mask = np.zeros(d, dtype=np.float64)
    mask[np.asarray(channels, dtype=np.int64)] = 1.0
    return mask


def pack_bits(bits: np.ndarray) -> np.ndarray:
    """Pack booleans [..., n] (n a multiple of 32) LSB-first: bit i of word w <- element 32 w + i."""
    n = bits.shape[-1]
    if n % 32:
        raise ValueError("bit count must be a multiple of 32")
    b = bits.reshape(*bits.shape[:-1], n // 32, 32).astype(np.uint64)
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    return (b * weights).sum(axis=-1).astype(np.uint32)


def unpack_bits(words: np.ndarray, n: int) -> np.ndarray:
    """Inverse of pack_bits: uint32 [..., n/32] -> bool [..., n]."""
    w = words.astype(np.uint64)[..., None]
    bits = (w >> np.arange(32, dtype=np.uint64)) & np.uint64(1)
    return bits.reshape(*words.shape[:-1], -1)[..., :n].astype(bool)


def pack_codes(codes: np.ndarray, nbits: int) -> np.ndarray:
    """Pack integer codes [..., d] into an LSB-first bit stream: code c occupies bits
    [nbits*c, nbits*c + nbits) of the row; returns uint8 [..., d*nbits/8]."""
    d = codes.shape[-1]
    if (d * nbits) % 8:
        raise ValueError("d * nbits must be a multiple of 8")
    c = codes.astype(np.uint64)[..., None]
    bits = ((c >> np.arange(nbits, dtype=np.uint64)) & np.uint64(1)).reshape(*codes.shape[:-1], d * nbits)
    b = bits.reshape(*codes.shape[:-1], d * nbits // 8, 8)
    return (b * (np.uint64(1) << np.arange(8, dtype=np.uint64))).sum(axis=-1).astype(np.uint8)


def unpack_codes(packed: np.ndarray, nbits: int, d: int) -> np.ndarray:
    """Inverse of pack_codes: uint8 [..., d*nbits/8] -> int64 codes [..., d]."""
    p = packed.astype(np.uint64)[..., None]
    bits = ((p >> np.arange(8, dtype=np.uint64)) & np.uint64(1)).reshape(*packed.shape[:-1], -1)
    b = bits[..., : d * nbits].reshape(*packed.shape[:-1], d, nbits)
    return (b * (np.uint64(1) << np.arange(nbits, dtype=np.uint64))).sum(axis=-1).astype(np.int64)


# ----------------------------------------------------------------------------- keys

def jl_project(S: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Gaussian JL transform S x of every vector x[..., :] (fp64) [QJL "Approach"]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(S, dtype=np.float64).T


def quantize_key_vectors(k: np.ndarray, S_in: np.ndarray, S_out: np.ndarray, channels) -> dict:
    """Quantize keys k [n, d] of one KV head whose outlier channel set is `channels`.

    [QJL "Approach"]: apply the JL transform, keep only the signs plus the key norm; outlier
    channels go through a separate quantizer copy.  Steps, per key:
      1. split k into its inlier part k_in = k * (1 - mask) and outlier part k_out = k * mask;
      2. p_in = S_in k_in (m values), p_out = S_out k_out (m_out values), fp64;
      3. sign bits: bit = 1 where p >= 0;
      4. pack: inlier words then outlier words, LSB-first;
      5. norms ||k_in||, ||k_out|| rounded to fp16 ("16-bit norm" [1BIT "But Wait"]).
    Also returns, for parity accounting, the near-zero flags |p_j| < 1e-5 * ||k|| (full key norm).
    """
    k = np.asarray(k, dtype=np.float64)
    n, d = k.shape
    mask = outlier_mask(d, channels)
    k_in = k * (1.0 - mask)
    k_out = k * mask
    p_in = jl_project(S_in, k_in)
    p_out = jl_project(S_out, k_out)
    p = np.concatenate([p_in, p_out], axis=1)
    bits = p >= 0.0
    words = pack_bits(bits)
    norms = np.stack([fp16(np.sqrt(np.sum(k_in * k_in, axis=1))),
                      fp16(np.sqrt(np.sum(k_out * k_out, axis=1)))], axis=1)
    full_norm = np.sqrt(np.sum(k * k, axis=1))
    near_zero = np.abs(p) < 1e-5 * full_norm[:, None]
    return {"bits": words, "norms": norms, "near_zero": near_zero, "proj": p}


def quantize_keys(K: np.ndarray, S_in: np.ndarray, S_out: np.ndarray, outlier_idx: np.ndarray) -> dict:
    """Keys in the model layout K [B, T, Hkv, d] -> cache layout.

    Returns bits [B, Hkv, T, (m + m_out)/32] uint32, norms [B, Hkv, T, 2] float16 (inlier, outlier)
    and near_zero [B, Hkv, T, m + m_out] bool.
    """
    B, T, Hkv, d = K.shape
    m, m_out = S_in.shape[0], S_out.shape[0]
    W = (m + m_out) // 32
    bits = np.zeros((B, Hkv, T, W), dtype=np.uint32)
    norms = np.zeros((B, Hkv, T, 2), dtype=np.float16)
    near = np.zeros((B, Hkv, T, m + m_out), dtype=bool)
    for b in range(B):
        for h in range(Hkv):
            r = quantize_key_vectors(K[b, :, h, :], S_in, S_out, outlier_idx[h] if outlier_idx.size else [])
            bits[b, h], norms[b, h], near[b, h] = r["bits"], r["norms"], r["near_zero"]
    return {"bits": bits, "norms": norms, "near_zero": near}


def select_outliers(K: np.ndarray, n_out: int) -> np.ndarray:
    """Outlier channels of every KV head from keys K [B, T, Hkv, d] -> int32 [Hkv, n_out].

    The pages describe outlier channels as the few coordinates whose magnitudes are 10-100x those of
    the rest [2NUM "The Real Problem: Outlier Channels"; HARD "The Third Problem: Magnitude
    Outliers": "detecting them"]; the detection statistic is not given.  Read here as the mean of
    |k_c| over the B*T keys of the head, in fp64; the n_out largest means win, the lower channel
    first on equal means, and the chosen channels are listed in ascending order.
    """
    K = np.asarray(K, dtype=np.float64)
    B, T, Hkv, d = K.shape
    out = np.zeros((Hkv, n_out), dtype=np.int32)
    for h in range(Hkv):
        mean_abs = np.abs(K[:, :, h, :]).reshape(B * T, d).mean(axis=0) if B * T else np.zeros(d)
        order = sorted(range(d), key=lambda c: (-mean_abs[c], c))      # largest mean, then lower channel
        out[h] = np.sort(np.array(order[:n_out], dtype=np.int32))
    return out


# ----------------------------------------------------------------------------- values

def quantize_value_vectors(v: np.ndarray, nbits: int) -> tuple[np.ndarray, np.ndarray]:
    """Token-wise min/max quantization of value vectors v [n, d] [QJL "Limitations": values use
    standard token-wise quantization; [2NUM "The Obvious Fix"]: find the range, divide it into 2^b
    equally spaced values, round to the nearest].

    IEEE float32 steps (the same decisions the kernel takes):
      mn = min v, mx = max v; step = fp16((mx - mn) / L) with L = 2^b - 1; mn16 = fp16(mn);
      code = clamp(rint((v - mn16) / step), 0, L)  (rint: ties to even), all codes 0 if step == 0.
    Returns (codes int64 [n, d], meta float16 [n, 2] = (mn16, step)).
    """
    v = np.asarray(v, dtype=np.float32)
    L = np.float32(2 ** nbits - 1)
    mn = v.min(axis=1)
    mx = v.max(axis=1)
    step16 = ((mx - mn) / L).astype(np.float16)
    mn16 = mn.astype(np.float16)
    step32 = step16.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((v - mn16.astype(np.float32)[:, None]) / step32)
    q = np.where(step32 == 0, np.float32(0), q)
    codes = np.clip(q, 0, L).astype(np.int64)
    return codes, np.stack([mn16, step16], axis=1)


def dequantize_value_vectors(codes: np.ndarray, meta: np.ndarray) -> np.ndarray:
    """v_hat = mn16 + step16 * code (fp64): the level the code names."""
    mn = meta[..., 0].astype(np.float64)[..., None]
    step = meta[..., 1].astype(np.float64)[..., None]
    return mn + step * codes.astype(np.float64)


def quantize_values(V: np.ndarray, nbits: int) -> dict:
    """Values in the model layout V [B, T, Hkv, d] -> codes [B, Hkv, T, d*nbits/8] uint8 and
    meta [B, Hkv, T, 2] float16."""
    B, T, Hkv, d = V.shape
    codes = np.zeros((B, Hkv, T, d * nbits // 8), dtype=np.uint8)
    meta = np.zeros((B, Hkv, T, 2), dtype=np.float16)
    for b in range(B):
        for h in range(Hkv):
            c, mt = quantize_value_vectors(V[b, :, h, :], nbits)
            codes[b, h] = pack_codes(c, nbits)
            meta[b, h] = mt
    return {"codes": codes, "meta": meta}


# ----------------------------------------------------------------------------- decode

def project_query(q: np.ndarray, S_in: np.ndarray, S_out: np.ndarray, channels) -> tuple[np.ndarray, np.ndarray]:
    """The query is JL-projected without quantization [QJL "Approach"]; it is split by the same
    outlier mask as the keys of its KV head: (S_in q_in, S_out q_out) in fp64."""
    q = np.asarray(q, dtype=np.float64)
    mask = outlier_mask(q.shape[-1], channels)
    return jl_project(S_in, q * (1.0 - mask)), jl_project(S_out, q * mask)


def estimator_scores(sq_in: np.ndarray, sq_out: np.ndarray, bits: np.ndarray, norms: np.ndarray) -> np.ndarray:
    """Asymmetric estimate of <q, k> for every key of one KV head.

    sq_in [m], sq_out [m_out]: the projected query; bits [n, W] and norms [n, 2] fp16 from the key
    quantizer.  score = sqrt(pi/2)/m * ||k_in|| * <S_in q_in, s_in> + sqrt(pi/2)/m_out * ||k_out|| *
    <S_out q_out, s_out>, with s = +1 for a set bit and -1 otherwise (the outlier term is absent when
    m_out = 0).  [QJL "Approach" and "Surprising findings": one side quantized to signs gives an
    unbiased inner-product estimate.]
    """
    m, m_out = sq_in.shape[0], sq_out.shape[0]
    n = bits.shape[0]
    score = np.zeros(n, dtype=np.float64)
    for t0 in range(0, n, _SLICE):          # independent keys, evaluated a slice at a time
        t1 = min(n, t0 + _SLICE)
        signs = np.where(unpack_bits(bits[t0:t1], m + m_out), 1.0, -1.0)
        n_in = norms[t0:t1, 0].astype(np.float64)
        n_out = norms[t0:t1, 1].astype(np.float64)
        s = SQRT_HALF_PI / m * n_in * (signs[:, :m] @ sq_in)
        if m_out:
            s = s + SQRT_HALF_PI / m_out * n_out * (signs[:, m:] @ sq_out)
        score[t0:t1] = s
    return score


def two_sided_scores(sq_in: np.ndarray, sq_out: np.ndarray, qn_in: float, qn_out: float, bits: np.ndarray,
                     norms: np.ndarray) -> np.ndarray:
    """Both sides quantized to signs, for every key of one KV head [QJL "Surprising findings"].

    sq_in [m], sq_out [m_out]: the projected query, of which only the signs are used (sign(0) = +1);
    qn_in, qn_out: the norms of the query's inlier and outlier parts; bits [n, W], norms [n, 2] fp16
    from the key quantizer.  score = qn_in * ||k_in|| / m * <sign(S_in q_in), s_in> + qn_out *
    ||k_out|| / m_out * <sign(S_out q_out), s_out>: the mean sign agreement of each part times both
    norms, a biased estimate of <q, k> (expectation ||q|| ||k|| (1 - 2 theta / pi) per part).
    """
    m, m_out = sq_in.shape[0], sq_out.shape[0]
    n = bits.shape[0]
    qs_in = np.where(sq_in >= 0, 1.0, -1.0)
    qs_out = np.where(sq_out >= 0, 1.0, -1.0)
    score = np.zeros(n, dtype=np.float64)
    for t0 in range(0, n, _SLICE):          # independent keys, evaluated a slice at a time
        t1 = min(n, t0 + _SLICE)
        signs = np.where(unpack_bits(bits[t0:t1], m + m_out), 1.0, -1.0)
        n_in = norms[t0:t1, 0].astype(np.float64)
        n_out = norms[t0:t1, 1].astype(np.float64)
        s = qn_in * n_in / m * (signs[:, :m] @ qs_in)
        if m_out:
            s = s + qn_out * n_out / m_out * (signs[:, m:] @ qs_out)
        score[t0:t1] = s
    return score


def rotate_sign_scores(q: np.ndarray, K: np.ndarray, R: np.ndarray) -> np.ndarray:
    """Rotate-then-sign keys [1BIT "The 1-Bit Breakthrough": sign after a rotation; "But Wait. Don't
    the Small Dims Overpower?": the norm is stored separately and the key is reconstructed as norm x
    signs]: for keys K [n, d] and an orthogonal R [d, d], the reconstruction ||k|| sign(R k) / sqrt(d)
    (scaled so that its norm is ||k||) dotted with the rotated query R q, in fp64 with the exact key
    norms; sign(0) = +1."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    d = R.shape[1]
    rq = R @ q
    rk = K @ R.T
    khat = np.linalg.norm(K, axis=1)[:, None] * np.where(rk >= 0, 1.0, -1.0) / math.sqrt(d)
    return khat @ rq


def softmax(z: np.ndarray) -> np.ndarray:
    """Two-pass softmax in fp64: subtract the max, exponentiate, normalise."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def attend(scores: np.ndarray, values: np.ndarray, sm_scale: float) -> np.ndarray:
    """o = sum_t softmax(sm_scale * s)_t v_t (fp64) [1BIT "Keys Select. Values Deliver."]."""
    if scores.shape[0] == 0:
        return np.zeros(values.shape[-1], dtype=np.float64)
    return softmax(sm_scale * scores) @ np.asarray(values, dtype=np.float64)


def decode_attention(Q: np.ndarray, S_in: np.ndarray, S_out: np.ndarray, outlier_idx: np.ndarray,
                     bits: np.ndarray, norms: np.ndarray, N: int, *, codes=None, meta=None,
                     V_f32=None, nbits: int = 2, sm_scale: float | None = None,
                     units=None, estimator: str = "one_sided") -> dict:
    """One decode step for every sequence and query head.

    Q [B, Hq, d]; bits [B, Hkv, >=N, W]; norms [B, Hkv, >=N, 2]; values either as codes
    [B, Hkv, >=N, d*nbits/8] + meta [B, Hkv, >=N, 2] or unquantized V_f32 [B, Hkv, >=N, d].
    Query head hq reads KV head hq // (Hq/Hkv).  sm_scale defaults to 1/sqrt(d).
    `units` optionally restricts the work to a list of (b, hq) pairs (others stay NaN).
    `estimator`: "one_sided" (the query unquantized, estimator_scores) or "two_sided" (the query
    reduced to its signs as well, two_sided_scores).
    Returns out [B, Hq, d] and scores [B, Hq, N] (raw estimator scores, before sm_scale), fp64.
    """
    if estimator not in ("one_sided", "two_sided"):
        raise ValueError(f"unknown estimator {estimator!r}")
    B, Hq, d = Q.shape
    Hkv = bits.shape[1]
    g = Hq // Hkv
    if sm_scale is None or sm_scale <= 0:
        sm_scale = 1.0 / math.sqrt(d)
    out = np.full((B, Hq, d), np.nan)
    scores = np.full((B, Hq, N), np.nan)
    todo = units if units is not None else [(b, hq) for b in range(B) for hq in range(Hq)]
    vcache = {}
    for b, hq in todo:
        h = hq // g
        channels = outlier_idx[h] if outlier_idx.size else []
        sq_in, sq_out = project_query(Q[b, hq], S_in, S_out, channels)
        if estimator == "one_sided":
            s = estimator_scores(sq_in, sq_out, bits[b, h, :N], norms[b, h, :N])
        else:
            q = np.asarray(Q[b, hq], dtype=np.float64)
            mask = outlier_mask(d, channels)
            qn_in, qn_out = float(np.linalg.norm(q * (1.0 - mask))), float(np.linalg.norm(q * mask))
            s = two_sided_scores(sq_in, sq_out, qn_in, qn_out, bits[b, h, :N], norms[b, h, :N])
        if (b, h) not in vcache:
            if V_f32 is not None:
                vcache[(b, h)] = np.asarray(V_f32[b, h, :N], dtype=np.float64)
            else:
                vcache[(b, h)] = dequantize_value_vectors(unpack_codes(codes[b, h, :N], nbits, d), meta[b, h, :N])
        out[b, hq] = attend(s, vcache[(b, h)], sm_scale)
        scores[b, hq] = s
    return {"out": out, "scores": scores}


def exact_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """Unquantized attention of one query over keys K [n, d] and values V [n, d] (reporting only)."""
    return attend(np.asarray(K, np.float64) @ np.asarray(q, np.float64), V, sm_scale)


# ----------------------------------------------------------------------------- baselines

def uniform_quantize(x, lo: float = -1.0, hi: float = 1.0, nbits: int = 2) -> tuple[np.ndarray, np.ndarray]:
    """Fixed-range uniform scalar quantizer [HARD "Just Round Everything"]: 2^b equal-width buckets
    over [lo, hi] (the last one closed on the right); a value is stored as its bucket index and
    reconstructed as the bucket midpoint.  Returns (bucket index, reconstruction)."""
    x = np.asarray(x, dtype=np.float64)
    nb = 2 ** nbits
    width = (hi - lo) / nb
    idx = np.clip(np.floor((x - lo) / width), 0, nb - 1).astype(np.int64)
    return idx, lo + (idx + 0.5) * width


def two_sided_estimate(q: np.ndarray, k: np.ndarray, S: np.ndarray) -> float:
    """Both sides quantized to signs: mean of sign(S q) * sign(S k), which estimates the
    angle-based quantity 1 - 2 theta/pi, not the cosine [QJL "Surprising findings"]."""
    sq = np.where(jl_project(S, q) >= 0, 1.0, -1.0)
    sk = np.where(jl_project(S, k) >= 0, 1.0, -1.0)
    return float(np.mean(sq * sk))
