"""Seeded synthetic inputs for the indexer top-k (shared by tests, bench and oracle checks).

This module only *creates* inputs: it draws random numbers and encodes them into
the byte formats the library consumes (OCP e4m3fn, OCP MXFP4 = e2m1 codes with
e8m0 block scales, bf16).  It holds none of the method's arithmetic: no scoring,
no decoding, no selection.  Both the HIP path and the CPU oracle read the same
bytes, so the encoders' rounding choices never affect parity.

Five workload families are provided (``make(cfg, ...)``):

1. ``tiny``     64 rows x 4096 keys, 32 heads, e4m3 integers in [-4, 4],
                integer head weights in [0, 3], causal, k = 512.
2. ``select``   selection only: 64 rows x 131072 fp32 scores ~ N(0, 0.05),
                30 % quantised to 2^-10 steps, a planted top band of 2048 values
                in runs of 32 keys, row lengths uniform in [2048, 131072].
3. ``prefill``  4096 rows x 65536 keys, 64 heads, e4m3 ~ N(0,1) with a per-key
                fp32 scale in [0.5, 2], w ~ U(0, 1/64), causal, k = 2048.
4. ``long``     4096 rows x 1,048,576 keys, 32 heads, MXFP4 of N(0,1) with the
                top keys planted in clustered runs of 16..64 keys, w ~ U(0,1/32).
5. ``decode``   128 requests x 4 MTP rows, context lengths log-uniform in
                [8192, 262144], K in 64-token pages behind a shuffled page table,
                e4m3 with a per-token scale, 64 heads, k = 2048.

Every family accepts smaller shapes (same distributions) for parity tests.
Random streams: ``numpy.random.SeedSequence(seed).spawn(n)``, one stream per
tensor; the default seed of family i is i - 1 for ``tiny`` (0) and i otherwise.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

HEAD_DIM = 128
PAGE = 64

FMT_E4M3 = "e4m3"
FMT_MXFP4 = "mxfp4"


@dataclasses.dataclass
class Problem:
    """Host-side (numpy) description of one indexer problem.

    Layouts (all C-contiguous):
      q      e4m3: uint8 [rows, H, 128];  mxfp4: uint8 [rows, H, 64] (element 2i in the low nibble)
      q_sf   mxfp4 only: uint8 [rows, H, 4] e8m0 scale of each 32-element block of head_dim
      k      contiguous: e4m3 uint8 [num_keys, 128] / mxfp4 uint8 [num_keys, 64]
             paged (e4m3 only): uint8 [num_pages, 64, 128]
      k_sf   mxfp4 only: uint8 [num_keys, 4]
      k_scale optional fp32 per key (contiguous) or per physical slot (paged)
      w      uint16 bf16 bits [rows, H]
      ks, ke int32 [rows]; row r sees keys [ks[r], ke[r]) (logical positions when paged)
      page_table int32 [num_req, max_pages] (paged only, -1 = unused)
      row_req int32 [rows] (paged only)
    """

    name: str
    fmt: str
    rows: int
    heads: int
    q: np.ndarray
    q_sf: Optional[np.ndarray]
    k: np.ndarray
    k_sf: Optional[np.ndarray]
    k_scale: Optional[np.ndarray]
    w: np.ndarray
    ks: np.ndarray
    ke: np.ndarray
    topk: int
    num_keys: int                      # contiguous: keys in k; paged: physical slots = num_pages * 64
    page_table: Optional[np.ndarray] = None
    row_req: Optional[np.ndarray] = None
    planted: Optional[np.ndarray] = None  # bool [num_keys] for the clustered family (reporting only)

    @property
    def paged(self) -> bool:
        return self.page_table is not None

    @property
    def pairs(self) -> int:
        """Visible (row, key) pairs = the algorithmic number of key-scores."""
        return int(np.sum(self.ke.astype(np.int64) - self.ks.astype(np.int64)))

    def row_slice(self, r0: int, r1: int) -> "Problem":
        """Rows [r0, r1) as a problem of their own (same K)."""
        def sl(a):
            return None if a is None else a[r0:r1]
        return dataclasses.replace(
            self, rows=r1 - r0, q=self.q[r0:r1], q_sf=sl(self.q_sf), w=self.w[r0:r1],
            ks=self.ks[r0:r1], ke=self.ke[r0:r1], row_req=sl(self.row_req))


@dataclasses.dataclass
class SelectProblem:
    """Selection-only input: fp32 rows of pitch ``ld``; row r uses x[r, :len[r]]."""

    name: str
    x: np.ndarray          # float32 [rows, ld]
    length: np.ndarray     # int32 [rows]
    topk: int

    @property
    def rows(self) -> int:
        return self.x.shape[0]


# --------------------------------------------------------------------------- encoders

def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """float -> OCP e4m3fn bytes, round-to-nearest-even, saturating at +-448."""
    t = torch.from_numpy(np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float -> bf16 bit patterns (uint16), round-to-nearest-even."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


# e2m1 codes 0..7 in magnitude order: 0, 0.5, 1, 1.5, 2, 3, 4, 6.  A magnitude maps to the
# nearer grid point; an exact midpoint goes to the neighbour whose mantissa bit is 0 (ties
# to even), which is why some edges below are strict (>) and others inclusive (>=).
def _e2m1_codes(y: np.ndarray) -> np.ndarray:
    a = np.abs(y)
    code = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0)).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << 3)


def encode_mxfp4(x: np.ndarray):
    """float [..., 128] -> (packed e2m1 uint8 [..., 64], e8m0 uint8 [..., 4]).

    OCP MX rule: per block of 32 consecutive elements the shared exponent is
    floor(log2(max|x|)) - 2 (2 = largest e2m1 exponent), elements are x / 2^e rounded
    to e2m1 (nearest, ties to even) and saturated at +-6.
    """
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] == HEAD_DIM
    lead = x.shape[:-1]
    xb = x.reshape(*lead, 4, 32)
    amax = np.max(np.abs(xb), axis=-1)
    _, ex = np.frexp(amax)                      # amax = m * 2^ex, m in [0.5, 1): floor(log2) = ex - 1
    e = np.where(amax > 0, ex.astype(np.int32) - 1 - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int32)
    y = np.ldexp(xb, (-e)[..., None].astype(np.int32)).astype(np.float32)   # exact power-of-two scaling
    codes = _e2m1_codes(y).reshape(*lead, HEAD_DIM)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    sf = (e + 127).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(sf)


# --------------------------------------------------------------------------- helpers

def _streams(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _causal(rows: int, num_keys: int):
    off = num_keys - rows
    ks = np.zeros(rows, dtype=np.int32)
    ke = (off + 1 + np.arange(rows)).astype(np.int32)
    return ks, ke


def _normal_e4m3(rng, shape, chunk=1 << 24):
    """N(0,1) -> e4m3 bytes, generated in chunks to bound host memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        out[i:i + m] = encode_e4m3(rng.standard_normal(m, dtype=np.float32))
    return out.reshape(shape)


# --------------------------------------------------------------------------- families

def tiny(rows=64, num_keys=4096, heads=32, topk=512, seed=0) -> Problem:
    rq, rk, rw = _streams(seed, 3)
    q = encode_e4m3(rq.integers(-4, 5, size=(rows, heads, HEAD_DIM)).astype(np.float32))
    k = encode_e4m3(rk.integers(-4, 5, size=(num_keys, HEAD_DIM)).astype(np.float32))
    w = encode_bf16(rw.integers(0, 4, size=(rows, heads)).astype(np.float32))
    ks, ke = _causal(rows, num_keys)
    return Problem("tiny", FMT_E4M3, rows, heads, q, None, k, None, None, w, ks, ke, topk, num_keys)


def prefill(rows=4096, num_keys=65536, heads=64, topk=2048, seed=3) -> Problem:
    rq, rk, rs, rw = _streams(seed, 4)
    q = _normal_e4m3(rq, (rows, heads, HEAD_DIM))
    k = _normal_e4m3(rk, (num_keys, HEAD_DIM))
    k_scale = rs.uniform(0.5, 2.0, size=num_keys).astype(np.float32)
    w = encode_bf16(rw.uniform(0.0, 1.0 / 64, size=(rows, heads)))
    ks, ke = _causal(rows, num_keys)
    return Problem("prefill", FMT_E4M3, rows, heads, q, None, k, None, k_scale, w, ks, ke, topk, num_keys)


def long_context(rows=4096, num_keys=1 << 20, heads=32, topk=2048, seed=4, band_keys=None) -> Problem:
    """MXFP4 family with the top keys clustered in runs of 16..64 keys.

    A shared unit vector u is added to every query head (2u) and to the planted keys
    (4u), so planted keys score high for every row.  Runs of U{16..64} keys are
    planted at random non-overlapping positions inside the range every row sees until
    about 2*topk keys are covered.
    """
    rq, rk, ru, rp, rw = _streams(seed, 5)
    u = ru.standard_normal(HEAD_DIM)
    u = (u / np.linalg.norm(u)).astype(np.float32)
    q = np.empty((rows, heads, HEAD_DIM // 2), dtype=np.uint8)
    q_sf = np.empty((rows, heads, 4), dtype=np.uint8)
    for i in range(0, rows, 512):
        m = min(512, rows - i)
        qf = rq.standard_normal((m, heads, HEAD_DIM), dtype=np.float32) + 2.0 * u
        q[i:i + m], q_sf[i:i + m] = encode_mxfp4(qf)
    ks, ke = _causal(rows, num_keys)
    common = int(ke.min())                       # keys [0, common) are visible to every row
    target = band_keys if band_keys is not None else 2 * topk
    planted = np.zeros(num_keys, dtype=bool)
    covered = 0
    slots = max(1, common // 64)
    order = rp.permutation(slots)                # one candidate run start per 64-key slot
    for s in order:
        if covered >= target:
            break
        ln = int(rp.integers(16, 65))
        start = int(s) * 64
        stop = min(start + ln, common)
        planted[start:stop] = True
        covered += stop - start
    k = np.empty((num_keys, HEAD_DIM // 2), dtype=np.uint8)
    k_sf = np.empty((num_keys, 4), dtype=np.uint8)
    chunk = 1 << 17
    for i in range(0, num_keys, chunk):
        m = min(chunk, num_keys - i)
        kf = rk.standard_normal((m, HEAD_DIM), dtype=np.float32)
        kf[planted[i:i + m]] += 4.0 * u
        k[i:i + m], k_sf[i:i + m] = encode_mxfp4(kf)
    w = encode_bf16(rw.uniform(0.0, 1.0 / 32, size=(rows, heads)))
    return Problem("long", FMT_MXFP4, rows, heads, q, q_sf, k, k_sf, None, w, ks, ke, topk,
                   num_keys, planted=planted)


def decode(num_req=128, q_len=4, ctx_lo=8192, ctx_hi=262144, heads=64, topk=2048, seed=5) -> Problem:
    """Paged e4m3 K behind a shuffled page table; q_len MTP rows per request.

    Context L of a request includes its q_len new tokens; row j (0-based) of the request
    sees logical keys [0, L - q_len + j], i.e. ke = L - q_len + j + 1.
    """
    rl, rperm, rq, rk, rs, rw = _streams(seed, 6)
    L = np.exp(rl.uniform(math.log(ctx_lo), math.log(ctx_hi), size=num_req)).astype(np.int64)
    L = np.maximum(L, q_len)
    pages_per = (L + PAGE - 1) // PAGE
    num_pages = int(pages_per.sum())
    max_pages = int(pages_per.max())
    perm = rperm.permutation(num_pages).astype(np.int32)
    page_table = np.full((num_req, max_pages), -1, dtype=np.int32)
    pos = 0
    for r in range(num_req):
        n = int(pages_per[r])
        page_table[r, :n] = perm[pos:pos + n]
        pos += n
    rows = num_req * q_len
    q = _normal_e4m3(rq, (rows, heads, HEAD_DIM))
    k = _normal_e4m3(rk, (num_pages, PAGE, HEAD_DIM))
    k_scale = rs.uniform(0.5, 2.0, size=num_pages * PAGE).astype(np.float32)
    w = encode_bf16(rw.uniform(0.0, 1.0 / 64, size=(rows, heads)))
    row_req = np.repeat(np.arange(num_req, dtype=np.int32), q_len)
    j = np.tile(np.arange(q_len), num_req)
    ks = np.zeros(rows, dtype=np.int32)
    ke = (L[row_req] - q_len + j + 1).astype(np.int32)
    return Problem("decode", FMT_E4M3, rows, heads, q, None, k, None, k_scale, w, ks, ke, topk,
                   num_pages * PAGE, page_table=page_table, row_req=row_req)


def select_only(rows=64, ld=131072, min_len=2048, topk=2048, seed=2, runs=64, run_len=32) -> SelectProblem:
    """fp32 rows ~ N(0, 0.05); 30 % of entries quantised to 2^-10 steps (dense ties);
    a planted band of runs*run_len values ~ N(0.2, 0.05) in runs of run_len keys."""
    rl, rx, rqz, rb, rv = _streams(seed, 5)
    length = rl.integers(min_len, ld + 1, size=rows).astype(np.int32)
    x = rx.normal(0.0, 0.05, size=(rows, ld)).astype(np.float32)
    for r in range(rows):
        n = int(length[r])
        slots = n // run_len
        pick = rb.choice(slots, size=min(runs, slots), replace=False)
        for s in pick:
            x[r, s * run_len:(s + 1) * run_len] = rv.normal(0.2, 0.05, size=run_len)
    qmask = rqz.random(size=(rows, ld)) < 0.30
    xq = (np.round(x.astype(np.float64) * 1024.0) / 1024.0).astype(np.float32)
    xq = np.where(np.signbit(x) & (xq == 0), np.float32(-0.0), xq)   # keep the sign of zeros
    x = np.where(qmask, xq, x).astype(np.float32)
    return SelectProblem("select", np.ascontiguousarray(x), length, topk)


@dataclasses.dataclass
class AttnProblem:
    """Inputs of the sparse attention consumer: q bf16 bits [rows, hq, 128], e4m3 K and V
    caches [num_slots, hkv, 128], selected physical slots int32 [rows, width] (-1 padded)."""
    name: str
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    slots: np.ndarray
    softmax_scale: float
    output_scale: float

    @property
    def rows(self):
        return self.q.shape[0]


def sparse_attn(rows=512, hq=24, hkv=2, width=2048, num_slots=262144, seed=6, short_every=16) -> AttnProblem:
    """Decode/verify rows attending to `width` selected slots each (the QSA page's shape:
    2048 selected tokens per row, 24 query heads over 2 KV heads, an fp8 e4m3 KV cache).
    q ~ N(0, 1) as bf16; K, V ~ N(0, 1) as e4m3; each row's slots are distinct, uniform over
    the cache.  Every `short_every`-th row keeps a random shorter selection (the rest -1) and
    the last row has none (a padding row).  softmax_scale = 1/sqrt(128), output_scale = 1."""
    rq, rk, rv, rs, rn = _streams(seed, 5)
    q = encode_bf16(rq.standard_normal((rows, hq, HEAD_DIM), dtype=np.float32))
    k = _normal_e4m3(rk, (num_slots, hkv, HEAD_DIM))
    v = _normal_e4m3(rv, (num_slots, hkv, HEAD_DIM))
    slots = np.empty((rows, width), dtype=np.int32)
    for r in range(rows):
        slots[r] = rs.choice(num_slots, size=width, replace=False)
        if short_every and r % short_every == short_every - 1:
            n = int(rn.integers(0, width + 1))
            slots[r, n:] = -1
    if rows:
        slots[rows - 1] = -1
    return AttnProblem("sparse_attn", q, k, v, slots, 1.0 / math.sqrt(HEAD_DIM), 1.0)


FAMILIES = {
    "tiny": tiny,
    "select": select_only,
    "prefill": prefill,
    "long": long_context,
    "decode": decode,
    "sparse_attn": sparse_attn,
}


def make(name: str, **kw):
    return FAMILIES[name](**kw)
