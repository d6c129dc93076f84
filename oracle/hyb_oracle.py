"""CPU oracle for the tile-hybrid dense / 2:4 weight format and its matmul.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's cpu_baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it, and it shares no code,
table or constant generator with that path.

Everything here is plain NumPy on 16-bit bit patterns (uint16) so that packing
and unpacking are defined bit for bit, and the matmul is done in float64 from
exact widenings of the 16-bit values.

What the method computes (sources cited by page title and section):

* PATCH: Learnable Tile-level Hybrid Sparsity for LLMs (gist.science),
  section 2 "Meccanismo Principale": the weight matrix is cut into b1 x b2
  tiles; each tile is either dense (nothing removed) or 2:4 sparse (half of
  the entries removed).  Section 2 "Distribuzioni Apprendibili": inside a
  sparse tile each group of four keeps one of the 6 possible two-of-four
  patterns.  Section 1 "Enunciato del Problema": a 2:4 group holds two
  non-zeros out of four consecutive entries.
* SparseDecoding (ai.info, authors' abstract): the N:M matrix is stored
  compressed and read through bitmask indexing with a fixed stride, i.e. a
  constant number of stored values per group.
* 3BASiL (gist.science), section 2 "Aggiornamenti Chiusi": projecting onto a
  sparsity set is magnitude pruning -- the rule used here to choose the two
  kept entries, since the pages' learned choice needs training data.

Readings where the pages are silent (each also listed in the design notes):
  R1 groups run along K (the input / reduction axis), 4 aligned columns;
  R2 the two kept entries are the two largest |w|, compared as the integer
     key bits & 0x7FFF, ties going to the lower position;
  R3 the two stored values are in ascending position order;
  R4 metadata nibble: idx2 = i0 | i1 << 2, mask4 = 1 << i0 | 1 << i1;
  R5 every group stores exactly two slots, zeros included;
  R6 dropped positions unpack to +0.0 (bit pattern 0x0000);
  R7 the stream layout below (format "HYB1");
  R8 ragged shapes (n % b1 or k % b2 non-zero) are rejected;
  R14 4:8 tiles (metadata kind "mask8"): PATCH section 5 "Significato"
      names 4:8 as the next N:M pattern and SparseDecoding's kernel serves
      N:M with bitmask indices.  Groups of eight aligned columns keep their
      four largest keys (R2's key and tie rule), stored in ascending
      position order, with an 8-bit mask (bit p set = position p kept).  A
      4:8 tile has the same byte counts as a 2:4 tile;
  R13 sparse + low-rank: L = U V^T (U n x r, V k x r) is held as its two
      factors and T = X V is computed before the product (ref_lowrank; T
      itself is ref_matmul of V^T and X).

Format HYB1 (all element indices count 16-bit words):
  tile t = tn * TK + tk, TN = n / b1, TK = k / b2, tile_map[tn, tk] in {0, 1};
  dense tiles take dense slots 0.. in increasing t, sparse tiles sparse
  slots 0.. in increasing t; tidx[t] = slot (dense) or ~slot (sparse).
  Dense slot s, local element (r, c):
      s*b1*b2 + (r//16)*16*b2 + (c//32)*512 + ((c%32)//8)*128 + (r%16)*8 + c%8
  Sparse slot s, row r, group g (columns 4g..4g+3), kept value j in {0, 1}:
      s*b1*b2/2 + (r//16)*8*b2 + (g//16)*512 + ((g%16)//4)*128 + (r%16)*8
      + (g%4)*2 + j
  Metadata (16-bit little-endian words), nibble of (s, r, g) sits in word
      s*b1*b2/16 + (r//16)*b2 + (((g%16)//4)*16 + r%16)*(b2//64) + g//16
  at bits 4*(g%4) .. 4*(g%4)+3.
  4:8 (mask8) sparse slot s, row r, group h (columns 8h..8h+7), kept value
  j in {0, 1, 2, 3}:
      s*b1*b2/2 + (r//16)*8*b2 + (h//8)*512 + ((h%8)//2)*128 + (r%16)*8
      + (h%2)*4 + j
  and its mask byte sits in the word of the 2:4 group g = 2h, at bits
  8*(h%2) .. 8*(h%2)+7 (the same 16 columns per lane and word as 2:4).
  Requires b1 % 16 == 0 and b2 % 64 == 0.
"""
from __future__ import annotations

import numpy as np

META_KINDS = ("idx2", "mask4", "mask8")
DTYPES = ("bf16", "f16")

# The six two-of-four patterns (PATCH section 2, "Distribuzioni Apprendibili"),
# as ascending position pairs.
PATTERNS = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]


# ---------------------------------------------------------------- values ----

def widen(bits, dtype: str) -> np.ndarray:
    """Exact float64 value of 16-bit patterns (fp16 or bf16)."""
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def magnitude_key(bits) -> np.ndarray:
    """R2: |w| as an integer.  For fp16 and bf16 alike, clearing the sign bit
    leaves an unsigned integer that grows with the magnitude of every finite
    value (subnormals included, +0 and -0 both 0); Inf sorts above every
    finite value and NaN above Inf."""
    return np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)


def kept_positions(group_bits) -> tuple[np.ndarray, np.ndarray]:
    """Positions (i0 < i1) of the two entries kept in each group of four.

    group_bits: uint16 array of shape (..., 4).  Entries are ranked by
    magnitude key, larger first, and among equal keys the lower position
    first (R2); the first two of that ranking are kept.
    """
    g = np.asarray(group_bits, dtype=np.uint16)
    key = magnitude_key(g).astype(np.int64)
    pos = np.arange(4, dtype=np.int64)
    # Larger key first; for equal keys the lower position first.
    rank_score = key * 4 + (3 - pos)
    order = np.argsort(-rank_score, axis=-1, kind="stable")
    first, second = order[..., 0], order[..., 1]
    return np.minimum(first, second), np.maximum(first, second)


def group_shape(meta: str) -> tuple[int, int]:
    """(kept, group size) of a sparse tile's groups: 2:4 for idx2 and mask4,
    4:8 for mask8 (R14)."""
    if meta in ("idx2", "mask4"):
        return 2, 4
    if meta == "mask8":
        return 4, 8
    raise ValueError(f"unknown metadata kind {meta!r}")


def kept_positions_nm(group_bits, keep: int) -> np.ndarray:
    """Ascending positions of the `keep` entries kept in each group.

    group_bits: uint16 array of shape (..., size).  The same rule as the
    2:4 case (R2): rank by magnitude key, larger first, equal keys by lower
    position; the first `keep` of the ranking are kept.  Returns int64
    (..., keep)."""
    g = np.asarray(group_bits, dtype=np.uint16)
    size = g.shape[-1]
    key = magnitude_key(g).astype(np.int64)
    pos = np.arange(size, dtype=np.int64)
    rank_score = key * size + (size - 1 - pos)
    order = np.argsort(-rank_score, axis=-1, kind="stable")
    return np.sort(order[..., :keep], axis=-1)


def mask8(positions) -> np.ndarray:
    """R14: 8-bit mask of a 4:8 group with kept positions (..., 4)."""
    p = np.asarray(positions, dtype=np.int64)
    return np.bitwise_or.reduce(np.left_shift(1, p), axis=-1).astype(np.uint8)


def positions_from_mask8(mask) -> np.ndarray:
    """Inverse of `mask8`; raises ValueError unless exactly four bits are set."""
    m = np.asarray(mask, dtype=np.int64)
    bits = (m[..., None] >> np.arange(8)) & 1
    if np.any(bits.sum(axis=-1) != 4):
        bad = np.unique(m[bits.sum(axis=-1) != 4])
        raise ValueError(f"invalid mask8 bytes: {bad.tolist()}")
    return np.argsort(1 - bits, axis=-1, kind="stable")[..., :4]


def nibble(i0, i1, meta: str) -> np.ndarray:
    """R4: metadata nibble of a group whose kept positions are i0 < i1."""
    i0 = np.asarray(i0, dtype=np.int64)
    i1 = np.asarray(i1, dtype=np.int64)
    if meta == "idx2":
        return (i0 | (i1 << 2)).astype(np.uint8)
    if meta == "mask4":
        return ((1 << i0) | (1 << i1)).astype(np.uint8)
    raise ValueError(f"unknown metadata kind {meta!r}")


def positions_from_nibble(nib, meta: str) -> tuple[np.ndarray, np.ndarray]:
    """Inverse of `nibble`; raises ValueError on a nibble outside the six
    valid patterns."""
    nib = np.asarray(nib, dtype=np.int64)
    i0 = np.full(nib.shape, -1, dtype=np.int64)
    i1 = np.full(nib.shape, -1, dtype=np.int64)
    for a, b in PATTERNS:
        hit = nib == int(nibble(a, b, meta))
        i0[hit] = a
        i1[hit] = b
    if np.any(i0 < 0):
        bad = np.unique(nib[i0 < 0])
        raise ValueError(f"invalid {meta} nibbles: {bad.tolist()}")
    return i0, i1


# ---------------------------------------------------------------- tiles -----

def check_shape(n: int, k: int, b1: int, b2: int) -> tuple[int, int]:
    if b1 <= 0 or b2 <= 0 or b1 % 16 or b2 % 64:
        raise ValueError(f"tile {b1}x{b2}: need b1 % 16 == 0 and b2 % 64 == 0")
    if n < 0 or k < 0 or n % b1 or k % b2:
        raise ValueError(f"shape {n}x{k} is not a whole number of {b1}x{b2} tiles (R8)")
    return n // b1, k // b2


def plan(n: int, k: int, b1: int, b2: int, tile_map) -> dict:
    """Tile slots and stream sizes (format HYB1)."""
    tn, tk = check_shape(n, k, b1, b2)
    m = np.asarray(tile_map, dtype=np.uint8).reshape(-1)
    if m.size != tn * tk:
        raise ValueError(f"tile map has {m.size} entries, need {tn * tk}")
    if np.any(m > 1):
        raise ValueError("tile map entries must be 0 (dense) or 1 (sparse)")
    tidx = np.zeros(m.size, dtype=np.int32)
    nd = ns = 0
    for t in range(m.size):
        if m[t]:
            tidx[t] = ~ns
            ns += 1
        else:
            tidx[t] = nd
            nd += 1
    return {
        "tiles_n": tn, "tiles_k": tk, "n_dense": nd, "n_sparse": ns, "tidx": tidx,
        "dense_elems": nd * b1 * b2, "val_elems": ns * b1 * b2 // 2,
        "meta_words": ns * b1 * b2 // 16,
        "dense_bytes": nd * b1 * b2 * 2, "val_bytes": ns * b1 * b2,
        "meta_bytes": ns * b1 * b2 // 8, "tidx_bytes": 4 * m.size,
    }


def _tile(w, tn, tk, b1, b2):
    return w[tn * b1:(tn + 1) * b1, tk * b2:(tk + 1) * b2]


def prune(w_bits, tile_map, b1: int, b2: int, meta: str = "idx2") -> np.ndarray:
    """W' = the tile-hybrid pruned weight, as uint16 bit patterns.

    Dense tiles are copied unchanged; in a sparse tile every row's aligned
    groups of four columns keep their two largest-magnitude entries and the
    other two become +0.0 (PATCH section 2 "Meccanismo Principale" and
    "Distribuzioni Apprendibili"; readings R1, R2, R6).  With meta "mask8"
    the groups are eight columns and keep four (R14).
    """
    keep, size = group_shape(meta)
    w = np.asarray(w_bits, dtype=np.uint16)
    n, k = w.shape
    tn_count, tk_count = check_shape(n, k, b1, b2)
    tmap = np.asarray(tile_map, dtype=np.uint8).reshape(tn_count, tk_count)
    out = w.copy()
    for tn in range(tn_count):
        for tk in range(tk_count):
            if not tmap[tn, tk]:
                continue
            groups = _tile(w, tn, tk, b1, b2).reshape(b1, b2 // size, size)
            kept = kept_positions_nm(groups, keep)
            pos = np.arange(size)
            keepm = (pos[None, None, :, None] == kept[..., None, :]).any(axis=-1)
            pruned = np.where(keepm, groups, np.uint16(0)).reshape(b1, b2)
            _tile(out, tn, tk, b1, b2)[...] = pruned
    return out


# Index maps of format HYB1, written out as in the module docstring.

def dense_index(s, r, c, b1: int, b2: int):
    return (s * b1 * b2 + (r // 16) * 16 * b2 + (c // 32) * 512
            + ((c % 32) // 8) * 128 + (r % 16) * 8 + c % 8)


def value_index(s, r, g, j, b1: int, b2: int):
    return (s * (b1 * b2 // 2) + (r // 16) * 8 * b2 + (g // 16) * 512
            + ((g % 16) // 4) * 128 + (r % 16) * 8 + (g % 4) * 2 + j)


def value_index8(s, r, h, j, b1: int, b2: int):
    return (s * (b1 * b2 // 2) + (r // 16) * 8 * b2 + (h // 8) * 512
            + ((h % 8) // 2) * 128 + (r % 16) * 8 + (h % 2) * 4 + j)


def meta_word_index(s, r, g, b1: int, b2: int):
    return (s * (b1 * b2 // 16) + (r // 16) * b2
            + (((g % 16) // 4) * 16 + r % 16) * (b2 // 64) + g // 16)


def pack(w_bits, tile_map, b1: int, b2: int, meta: str) -> dict:
    """Compressed streams of W (format HYB1).

    Returns dict(dense=uint16[], val=uint16[], meta=uint8[] (little-endian
    16-bit words), tidx=int32[], plan=...).  Dense tiles are copied; for each
    sparse group the two kept values are stored in ascending position order
    with their nibble (SparseDecoding abstract: bitmask indexing, fixed
    stride; readings R3-R5, R7).  With meta "mask8" each group of eight
    stores its four kept values and a mask byte (R14).
    """
    if meta not in META_KINDS:
        raise ValueError(f"unknown metadata kind {meta!r}")
    w = np.asarray(w_bits, dtype=np.uint16)
    n, k = w.shape
    p = plan(n, k, b1, b2, tile_map)
    dense = np.zeros(p["dense_elems"], dtype=np.uint16)
    val = np.zeros(p["val_elems"], dtype=np.uint16)
    words = np.zeros(p["meta_words"], dtype=np.uint16)
    r = np.arange(b1)[:, None]
    c = np.arange(b2)[None, :]
    g = np.arange(b2 // 4)[None, :]
    tk_count = p["tiles_k"]
    for t, ti in enumerate(p["tidx"]):
        tn, tk = divmod(t, tk_count)
        tile = _tile(w, tn, tk, b1, b2)
        if ti >= 0:
            dense[dense_index(int(ti), r, c, b1, b2)] = tile
            continue
        s = int(~ti)
        if meta == "mask8":
            groups8 = tile.reshape(b1, b2 // 8, 8)
            kept = kept_positions_nm(groups8, 4)
            h = np.arange(b2 // 8)[None, :]
            for j in range(4):
                val[value_index8(s, r, h, j, b1, b2)] = np.take_along_axis(groups8, kept[..., j:j + 1], axis=-1)[..., 0]
            byte = mask8(kept).astype(np.uint16) << (8 * (h % 2)).astype(np.uint16)
            np.bitwise_or.at(words, meta_word_index(s, r, 2 * h, b1, b2), byte)
            continue
        groups = tile.reshape(b1, b2 // 4, 4)
        i0, i1 = kept_positions(groups)
        v0 = np.take_along_axis(groups, i0[..., None], axis=-1)[..., 0]
        v1 = np.take_along_axis(groups, i1[..., None], axis=-1)[..., 0]
        val[value_index(s, r, g, 0, b1, b2)] = v0
        val[value_index(s, r, g, 1, b1, b2)] = v1
        nib = nibble(i0, i1, meta).astype(np.uint16) << (4 * (g % 4)).astype(np.uint16)
        np.bitwise_or.at(words, meta_word_index(s, r, g, b1, b2), nib)
    return {"dense": dense, "val": val, "meta": words.astype("<u2").view(np.uint8),
            "tidx": p["tidx"], "plan": p}


def unpack(dense, val, meta_bytes, tidx, n: int, k: int, b1: int, b2: int, meta: str) -> np.ndarray:
    """W' from the compressed streams: dense tiles gathered back, sparse
    groups rebuilt from their two values and nibble (four values and mask
    byte for mask8), +0.0 elsewhere (R6)."""
    tn_count, tk_count = check_shape(n, k, b1, b2)
    tidx = np.asarray(tidx, dtype=np.int32).reshape(-1)
    if tidx.size != tn_count * tk_count:
        raise ValueError("tidx size does not match the tile grid")
    dense = np.asarray(dense, dtype=np.uint16)
    val = np.asarray(val, dtype=np.uint16)
    words = np.asarray(meta_bytes, dtype=np.uint8).view("<u2").astype(np.uint16)
    out = np.zeros((n, k), dtype=np.uint16)
    r = np.arange(b1)[:, None]
    c = np.arange(b2)[None, :]
    g = np.arange(b2 // 4)[None, :]
    for t, ti in enumerate(tidx):
        tn, tk = divmod(t, tk_count)
        dst = _tile(out, tn, tk, b1, b2)
        if ti >= 0:
            dst[...] = dense[dense_index(int(ti), r, c, b1, b2)]
            continue
        s = int(~ti)
        if meta == "mask8":
            h = np.arange(b2 // 8)[None, :]
            byte = (words[meta_word_index(s, r, 2 * h, b1, b2)] >> (8 * (h % 2)).astype(np.uint16)) & 0xFF
            kept = positions_from_mask8(byte)
            groups8 = np.zeros((b1, b2 // 8, 8), dtype=np.uint16)
            for j in range(4):
                np.put_along_axis(groups8, kept[..., j:j + 1], val[value_index8(s, r, h, j, b1, b2)][..., None],
                                  axis=-1)
            dst[...] = groups8.reshape(b1, b2)
            continue
        nib = (words[meta_word_index(s, r, g, b1, b2)] >> (4 * (g % 4)).astype(np.uint16)) & 0xF
        i0, i1 = positions_from_nibble(nib, meta)
        v0 = val[value_index(s, r, g, 0, b1, b2)]
        v1 = val[value_index(s, r, g, 1, b1, b2)]
        groups = np.zeros((b1, b2 // 4, 4), dtype=np.uint16)
        np.put_along_axis(groups, i0[..., None], v0[..., None], axis=-1)
        np.put_along_axis(groups, i1[..., None], v1[..., None], axis=-1)
        dst[...] = groups.reshape(b1, b2)
    return out


# ---------------------------------------------------------------- matmul ----

def ref_matmul(wp_bits, x_bits, dtype: str) -> tuple[np.ndarray, np.ndarray]:
    """y_ref[m, n] = sum_k W'[n, k] X[m, k] and s[m, n] = sum_k |W'[n, k] X[m, k]|,
    both in float64 from exact widenings (the hybrid product equals the plain
    product with the pruned weight: compression only skips stored zeros,
    SparseDecoding abstract)."""
    w = widen(wp_bits, dtype)
    x = widen(np.atleast_2d(np.asarray(x_bits, dtype=np.uint16)), dtype)
    return x @ w.T, np.abs(x) @ np.abs(w).T


def ref_lowrank(wp_bits, x_bits, t, u_bits, dtype: str) -> tuple[np.ndarray, np.ndarray]:
    """Sparse + low-rank product (3BASiL, gist.science, section 1 "Il
    Problema": W ~ S + L with L of rank r; section 4 "Risultati
    Sperimentali": 2:4 sparse + rank 64).  With S = W' (the hybrid weight)
    and L = U V^T held as its factors (U n x r, V k x r), and T = X V
    given (float32, m x r):

        y_ref[m, n] = sum_k W'[n, k] X[m, k] + sum_j T[m, j] U[n, j]
        s[m, n]     = sum_k |W'[n, k] X[m, k]| + sum_j |T[m, j] U[n, j]|

    in float64 from exact widenings (T is taken as given, so the check does
    not depend on how T was rounded).  R13: L enters through its factors and
    T is computed before the product."""
    y, s = ref_matmul(wp_bits, x_bits, dtype)
    tt = np.atleast_2d(np.asarray(t, dtype=np.float64))
    uu = widen(np.atleast_2d(np.asarray(u_bits, dtype=np.uint16)), dtype)
    return y + tt @ uu.T, s + np.abs(tt) @ np.abs(uu).T


def ref_rows(wp_bits, x_bits, dtype: str, rows) -> tuple[np.ndarray, np.ndarray]:
    """`ref_matmul` restricted to the output columns n in `rows`."""
    rows = np.asarray(rows, dtype=np.int64)
    return ref_matmul(np.asarray(wp_bits)[rows], x_bits, dtype)


def within_bound(y, y_ref, s, rel: float = 2e-3, extra=0.0) -> np.ndarray:
    """Acceptance: |y - y_ref| <= rel * s (+ extra, e.g. half an output ulp)."""
    y = np.asarray(y, dtype=np.float64)
    return np.abs(y - y_ref) <= rel * s + extra


def sparsity(tile_map, b1: int, b2: int, n: int, k: int) -> float:
    """Fraction of dropped positions: half of every sparse tile (PATCH
    section 2: a dense tile keeps all entries, a 2:4 tile half of them)."""
    ns = int(np.asarray(tile_map).sum())
    return 0.5 * ns * b1 * b2 / (n * k) if n * k else 0.0
