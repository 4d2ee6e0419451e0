"""Plain CPU oracle for the DSA lightning-indexer top-k.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may.  It shares no code with the HIP library (no decoders, tables,
helpers or constants are shared); the two meet only at the input bytes produced by
``sparse_attention_indexer_score_amd.workloads``.

What it computes, and where that is defined
-------------------------------------------
* The indexer of DeepSeek Sparse Attention scores every key a query row can see and
  keeps the top ``k`` (512..2048) keys for attention (LiteTopK prefill indexer page,
  sgl-project/sglang#47469, introduction).  The score is the MQA "logits" of
  DeepGEMM's ``mqa_logits`` (same page, introduction): per query head h a dot product
  of that head's query with the key's single shared vector, ReLU, then a sum over
  heads weighted by the per-row head weight (same page, section 1: each thread of the
  scoring tile holds one key and sums its heads in registers):

      score[r, s] = kscale[s] * sum_h w[r, h] * max(q[r, h] . k[s], 0)

  computed here in float64 from exactly decoded inputs and rounded once to fp32.
* The top-k is exact (ROCm DSA indexer top-k page, sgl-project/sglang#37591, code
  analysis: an fp32 coarse histogram and a rescan on tie-buffer overflow give recall 1.0,
  as torch.topk does): order by fp32
  value descending (-0.0 == +0.0), ties broken by the lower key index, keep
  min(k, visible) indices relative to the row's first visible key, pad with -1.
* Paged K (LiteTopK page, section 3, topk_page_table_transform): logical position s of
  a request lives in physical slot page_table[req][s // 64] * 64 + s % 64.
* The consumer of the selection, sparse attention of each query row over its selected KV
  slots (QSA sparse paged attention page, vllm-project/vllm#66512): softmax of the scaled
  q . k over the selected slots, weights applied to the slots' value vectors
  (``sparse_attention``).

Readings where the pages are silent:
* e4m3 is OCP E4M3FN (bias 7, no infinities, 0x7F/0xFF NaN); MXFP4 is OCP e2m1 with
  one e8m0 scale per 32 consecutive head_dim elements, element 2i in the low nibble.
* A per-key fp32 scale multiplies the decoded key vector (equivalently the score,
  since ReLU(c x) = c ReLU(x) for c > 0).
* NaN inputs are rejected (ValueError).

Exactness: e4m3 and MXFP4 products are exact in float64 and a 128-term dot of them
fits in 53 bits, so every per-head dot is exact; the weighted head sum and the scale
product add at most a few 2^-53 relative, so the fp32 result is the correctly rounded
real score except in double-rounding corner cases (far below the fp32 tolerance).
"""
from __future__ import annotations

import numpy as np

PAGE = 64
HEAD_DIM = 128


# --------------------------------------------------------------------------- decoders

def _e4m3fn_value(b: int) -> float:
    """OCP E4M3FN: sign | 4-bit exponent (bias 7) | 3-bit mantissa; e=0 subnormal m*2^-9."""
    s = -1.0 if (b >> 7) & 1 else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _e2m1_value(n: int) -> float:
    """OCP e2m1: sign | 2-bit exponent (bias 1) | 1-bit mantissa; e=0 subnormal m*0.5."""
    s = -1.0 if (n >> 3) & 1 else 1.0
    e = (n >> 1) & 0x3
    m = n & 0x1
    if e == 0:
        return s * m * 0.5
    return s * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def _e8m0_value(b: int) -> float:
    """OCP e8m0 scale: 2^(b - 127); 0xFF is NaN."""
    return float("nan") if b == 0xFF else 2.0 ** (b - 127)


E4M3_TABLE = np.array([_e4m3fn_value(b) for b in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([_e2m1_value(n) for n in range(16)], dtype=np.float64)
E8M0_TABLE = np.array([_e8m0_value(b) for b in range(256)], dtype=np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    return E8M0_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an IEEE fp32 pattern."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):                           # NaN patterns stay NaN
        return u32.view(np.float32).astype(np.float64)


def decode_mxfp4(packed: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """uint8 [..., 64] (two e2m1 per byte, element 2i low) + e8m0 [..., 4] -> float64 [..., 128]."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = E2M1_TABLE[packed & 0xF]
    hi = E2M1_TABLE[packed >> 4]
    vals = np.empty(packed.shape[:-1] + (HEAD_DIM,), dtype=np.float64)
    vals[..., 0::2] = lo
    vals[..., 1::2] = hi
    scale = decode_e8m0(sf)                                   # [..., 4]
    vals = vals.reshape(packed.shape[:-1] + (4, 32)) * scale[..., None]
    return vals.reshape(packed.shape[:-1] + (HEAD_DIM,))


def _check_finite(a: np.ndarray, what: str):
    if not np.all(np.isfinite(a)):
        raise ValueError(f"{what}: NaN code in input")


# --------------------------------------------------------------------------- inputs

def dequant_q(p, rows=None) -> np.ndarray:
    """Query heads of the given rows as float64 [n, H, 128]."""
    rows = np.arange(p.rows) if rows is None else np.asarray(rows)
    if p.fmt == "e4m3":
        q = decode_e4m3(p.q[rows])
    else:
        q = decode_mxfp4(p.q[rows], p.q_sf[rows])
    _check_finite(q, "q")
    return q


def physical_keys(p, r: int) -> np.ndarray:
    """Physical key index of every key row r sees, in logical order ks[r] .. ke[r]-1."""
    s = np.arange(int(p.ks[r]), int(p.ke[r]), dtype=np.int64)
    if p.page_table is None:
        return s
    prow = p.page_table[int(p.row_req[r])].astype(np.int64)
    return prow[s // PAGE] * PAGE + s % PAGE


def dequant_keys(p, phys: np.ndarray) -> np.ndarray:
    """Key vectors (times the optional per-key scale) as float64 [n, 128]."""
    if p.fmt == "e4m3":
        kc = p.k.reshape(-1, HEAD_DIM)[phys]
        kv = decode_e4m3(kc)
    else:
        kv = decode_mxfp4(p.k[phys], p.k_sf[phys])
    _check_finite(kv, "k")
    if p.k_scale is not None:
        kv = kv * p.k_scale[phys].astype(np.float64)[:, None]
    return kv


def all_keys(p) -> np.ndarray:
    """Every key of a contiguous problem, decoded once: float64 [num_keys, 128]
    (in slices of 16384 keys, which only bounds the size of the temporaries)."""
    out = np.empty((p.num_keys, HEAD_DIM), dtype=np.float64)
    step = 1 << 14
    for i in range(0, p.num_keys, step):
        j = min(p.num_keys, i + step)
        out[i:j] = dequant_keys(p, np.arange(i, j, dtype=np.int64))
    return out


def row_scores(p, r: int, qd=None, kd_all=None) -> np.ndarray:
    """fp32 scores of row r over its visible keys (index 0 = key ks[r]).

    ``kd_all`` (contiguous problems only) is ``all_keys(p)``, passed to avoid decoding K
    again for every row; it changes nothing in the arithmetic.
    """
    qr = dequant_q(p, [r])[0] if qd is None else qd              # [H, 128]
    w = decode_bf16(p.w[r])                                       # [H]
    phys = physical_keys(p, r)
    if kd_all is None:
        kv = dequant_keys(p, phys)                                # [V, 128]
    else:
        kv = kd_all[int(p.ks[r]):int(p.ke[r])]                    # contiguous: same rows, no copy
    dots = qr @ kv.T                                              # [H, V]  exact per head
    score = w @ np.maximum(dots, 0.0)                             # [V]
    return score.astype(np.float32)                               # one rounding to fp32


# --------------------------------------------------------------------------- selection

def select_topk(x: np.ndarray, k: int) -> np.ndarray:
    """Exact top-k of one fp32 row: value descending, ties to the lower index.

    Returns int32 [k]: the first min(k, len) entries are indices, the rest -1.  The
    comparison is numeric, so -0.0 and +0.0 are equal and tie by index.
    """
    x = np.asarray(x, dtype=np.float32)
    if np.any(np.isnan(x)):
        raise ValueError("NaN score")
    order = np.argsort(-x, kind="stable")          # stable: equal values keep index order
    n = min(k, x.shape[0])
    out = np.full(k, -1, dtype=np.int32)
    out[:n] = order[:n]
    return out


def select_rows(x: np.ndarray, length: np.ndarray, k: int, row_start=None) -> np.ndarray:
    """Top-k of each row of a materialised fp32 matrix; row r uses
    x[r, row_start[r] : row_start[r] + length[r]] and returns indices relative to row_start."""
    rows = x.shape[0]
    out = np.empty((rows, k), dtype=np.int32)
    for r in range(rows):
        s0 = 0 if row_start is None else int(row_start[r])
        out[r] = select_topk(x[r, s0:s0 + int(length[r])], k)
    return out


def topk(p, k=None, rows=None) -> np.ndarray:
    """Full oracle: exact top-k key indices (relative to ks[r]) for the given rows."""
    k = p.topk if k is None else k
    rows = list(range(p.rows) if rows is None else rows)
    kd_all = all_keys(p) if p.page_table is None else None
    out = np.empty((len(rows), k), dtype=np.int32)
    for i, r in enumerate(rows):
        out[i] = select_topk(row_scores(p, r, kd_all=kd_all), k)
    return out


def selected_value_recall(x: np.ndarray, idx: np.ndarray, k: int) -> float:
    """|multiset(values at idx) & multiset(top-min(k,n) values)| / min(k,n) for one row."""
    x = np.asarray(x, dtype=np.float32)
    n = min(k, x.shape[0])
    if n == 0:
        return 1.0
    got = np.sort(x[idx[idx >= 0]].astype(np.float64))[::-1]
    best = np.sort(x.astype(np.float64))[::-1][:n]
    # multiset intersection of two descending lists
    i = j = hit = 0
    while i < len(got) and j < n:
        if got[i] == best[j]:
            hit += 1
            i += 1
            j += 1
        elif got[i] > best[j]:
            i += 1
        else:
            j += 1
    return hit / n


def page_transform(idx: np.ndarray, page_row: np.ndarray) -> np.ndarray:
    """Logical request position -> physical KV slot with 64-token pages; -1 passes through
    (LiteTopK page, section 3)."""
    idx = np.asarray(idx, dtype=np.int64)
    out = np.where(idx >= 0, page_row[np.maximum(idx, 0) // PAGE].astype(np.int64) * PAGE + idx % PAGE, -1)
    return out.astype(np.int32)


# ------------------------------------------------------------ sparse attention (consumer)

def sparse_attention(q_bits: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, slots: np.ndarray,
                     softmax_scale: float, output_scale: float) -> np.ndarray:
    """Attention of each query row over only the KV slots its indexer selected (the consumer
    of the top-k: QSA sparse paged attention page, vllm-project/vllm#66512, introduction
    and section 2: every query row attends to about 2048 tokens chosen by the indexer; the
    logical -> physical slot translation is a separate pass, so this takes physical slots).

    q_bits  uint16 bf16 [rows, hq, 128]
    k_cache, v_cache  uint8 e4m3 [num_slots, hkv, 128] (one vector per slot and KV head)
    slots   int32 [rows, width]: physical slots; entries outside [0, num_slots) (e.g. the
            -1 padding of a short selection) take no part
    Query head h reads KV head h // (hq // hkv) (grouped query heads share a KV head).

        s_j      = softmax_scale * q[r, h] . k[slot_j, g]
        out[r,h] = output_scale * sum_j exp(s_j - max s) v[slot_j, g] / sum_j exp(s_j - max s)

    over the valid j; a row with no valid slot gives 0.  Computed in float64 from exactly
    decoded inputs (bf16 and e4m3 values are exact in float64), returned as float64."""
    q = decode_bf16(q_bits)
    kd = decode_e4m3(k_cache)
    vd = decode_e4m3(v_cache)
    _check_finite(q, "q")
    _check_finite(kd, "k_cache")
    _check_finite(vd, "v_cache")
    rows, hq, d = q.shape
    num_slots, hkv, _ = kd.shape
    group = hq // hkv
    out = np.zeros((rows, hq, d), dtype=np.float64)
    for r in range(rows):
        sl = np.asarray(slots[r], dtype=np.int64)
        sl = sl[(sl >= 0) & (sl < num_slots)]
        if sl.size == 0:
            continue
        for h in range(hq):
            g = h // group
            s = softmax_scale * (kd[sl, g, :] @ q[r, h, :])
            p = np.exp(s - s.max())
            out[r, h, :] = output_scale * (p @ vd[sl, g, :]) / p.sum()
    return out
