"""Plain CPU oracle of the Video Sparse Attention (VSA) hot path, in float64.

TEST INFRASTRUCTURE. This module is the checker, not the product: only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it. It shares no code with the HIP path (no kernels, headers,
helpers, tables or constants) and imports nothing from it.

What it computes, and where the pages define it:

* ``tile`` / ``untile`` -- cube tiling of the (T, H, W) latent grid into
  4x4x4 = 64-token cubes, cube-major, each cube padded to 64 slots, with the
  real-token count per cube (``vbs``).
  Pages: "Wan2.2 Production Values -- VSA Block-Sparse Attention Inputs +
  Reference", section "Shapes" (S_padded = 624 cubes x 64, 21x30x52 real tokens,
  624 = ceil(21/4) ceil(30/4) ceil(52/4)) and section "Operator contract"
  (attend only the first vbs[c] of 64); "VSA: Accelerating Video Diffusion
  Inference with Sparse Attention on AMD GPUs", section "Two-Stage
  Architecture", Stage 1 ((Ct, Ch, Cw) = (4, 4, 4) cubes of 64 tokens);
  "FastVideo Guide: Sliding Tile Attention", section "Implementation" (tile
  index it*(n_h*n_w) + ih*n_w + iw and the inverse permutation).
* ``mean_pool`` / ``cube_scores`` / ``topk_select`` -- the coarse selector:
  mean-pool q and k per cube, score cube against cube with a dot product, keep
  the top-k key cubes per query cube.
  Pages: VSA blog, "Two-Stage Architecture" Stage 1 and "Generating Sparsity
  Patterns" (einsum of pooled blocks, then torch.topk over the last axis);
  "Optimizing block-sparse INT8 attention and multi-expert step caching for
  Wan 2.2", section "Decoupling Block Selection from Sparse CUDA Kernels"
  (mean-pool summaries, dot-product block scores).
* ``select_cdf`` -- the selector with a cumulative-mass threshold: per row the
  cubes in score order, and the count of leading cubes whose softmax mass
  (scores times sm_scale) first reaches tau, capped at max_k.
  Pages: Wan INT8 blog, section "Decoupling Block Selection from Sparse CUDA
  Kernels" (sort the block scores per query block, keep key blocks by a
  cumulative distribution threshold).
* ``fwd`` -- the fine stage: for every (batch, head, query cube) and each of
  its 64 rows, softmax((q . K_sel^T) / sqrt(D)) . V_sel over the real tokens of
  the selected key/value cubes.
  Pages: dataset card, "Operator contract"; VSA blog, "Two-Stage Architecture"
  Stage 2 and "Sparse Traversal".
* ``fwd_lut`` -- the same over the first valid_block_num[b, h, c] entries of
  each index row, with two per-row statistics: the log-sum-exp of the scaled
  scores and max_prob = 1 / l, l = sum_j exp(s_j - max_i s_i).
  Pages: VSA blog, "Block-Sparse Encoding" (kv_block_idx + valid_block_num)
  and "Sparse Traversal" (the kernel loops over valid_block_num[query_block]
  entries); Wan INT8 blog, "Dynamic Sparsity Budgeting via Softmax
  Normalizer Registers" (max_prob = 1 / l_i).

* ``cube_order`` (with ``tile(..., order)``) and ``mask_to_lut`` -- the
  space-filling-curve cube order, and the conversion of a block relation
  matrix into the lookup table.
  Pages: VSA blog, "Two-Stage Architecture" (pre-stage: 3D space-filling
  curve reordering) and "Sparse Encoding in CK Tile" (Jenga's full M x M
  block matrix versus VSA's id list with a valid count).
* ``coarse_output`` / ``gated_combine`` -- the coarse stage's own output,
  attention among the mean-pooled cubes softmax(Qc Kc^T * sm_scale) Vc per
  (batch, head), and the layer output that mixes it with the fine output
  through gates: out = g_c * Oc[cube of the row] + g_f * O_fine.
  Pages: VSA blog, "Two-Stage Architecture" (Stage 1 works on mean-pooled
  cubes; the final output combines the coarse-stage and fine-stage outputs
  through learnable gates) and its VSA/Jenga comparison (a learnable gate
  between coarse and fine).

Readings where the pages are silent (each one is listed with its reason in
the design notes of the repository):

1. Cubes are numbered row-major over the cube grid: c = (ct*Nh + ch)*Nw + cw.
2. Inside a cube the real tokens come first, row-major over the cube's clipped
   extent (et, eh, ew); slots u >= vbs[c] are padding.
3. ``tile`` writes zeros into padding slots.
4. The mean-pool divides by vbs[c] (real tokens only).
5. Scores are raw dot products: no scale and no softmax (neither changes the
   per-row ranking).
6. Top-k order: score descending, equal scores by ascending cube id.
7. Padding query rows are computed exactly like real rows.
8. sm_scale defaults to 1/sqrt(D).
9. ``topk_idx`` rows hold distinct ids in [0, Nkv) (asserted).
10. A row whose selected cubes hold no real token outputs 0 (and, in
    ``fwd_lut``, lse = -inf and max_prob = 0).
11. The log-sum-exp is natural-log, over the scaled scores sm_scale q.k_j.
12. The cumulative distribution of ``select_cdf`` is that of the softmax of
    the row's cube scores times sm_scale (default 1/sqrt(D)); the count is the
    smallest n >= 1 whose leading n cubes hold at least tau of the mass.
13. The coarse output is dense attention of every pooled query cube over the
    pooled key cubes that hold a real token (vbs[j] > 0), with sm_scale
    (default 1/sqrt(D)); a row with no such key cube is 0. It is broadcast to
    the 64 rows of its cube.
14. The gates are given tensors of the output's shape, applied elementwise;
    how a model computes them (learned projections) is outside the path.
15. The space-filling curve orders whole 4x4x4 cubes (each block is then a
    compact region by construction); the curve is the 3D Hilbert curve of
    the power-of-two box holding the cube grid, restricted to the grid.
16. mask_to_lut keeps a row's lowest max_kv ids when more cells are set.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "CUBE",
    "decode_bf16",
    "round_to_bf16",
    "cube_grid",
    "cube_sizes",
    "slot_tokens",
    "tile",
    "untile",
    "hilbert_index_3d",
    "cube_order",
    "mask_to_lut",
    "mean_pool",
    "cube_scores",
    "topk_select",
    "select",
    "cdf_counts",
    "select_cdf",
    "fwd_unit",
    "fwd",
    "fwd_units",
    "fwd_unit_stats",
    "fwd_lut",
    "coarse_output",
    "gated_combine",
]

#: tokens per cube edge (the VSA blog: (Ct, Ch, Cw) = (4, 4, 4))
EDGE = 4
#: tokens per cube
CUBE = EDGE * EDGE * EDGE


# ----------------------------------------------------------------- bf16 values

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact).

    A bf16 value is the upper half of an IEEE binary32 value.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    The outputs of the operator are bf16 (dataset card, "Operator contract" and
    "Scoring / loss"), so the GPU output is compared with the oracle's float64
    result rounded this way. bf16 keeps 8 significant bits and the binary32
    exponent range (normal exponents -126..127, subnormal spacing 2^-133).
    Rounding is done in one step from float64 (no double rounding via float32).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(np.abs(xf))        # |x| = m 2^e, m in [0.5, 1)
    e = np.maximum(e - 1, -126)         # exponent of the leading bit, >= emin
    spacing = np.ldexp(1.0, e - 7)      # 8 significant bits
    r = np.rint(xf / spacing) * spacing  # exact scaling; rint ties to even
    r[np.abs(r) >= 2.0 ** 128] = np.inf * np.sign(r[np.abs(r) >= 2.0 ** 128])
    out[fin] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


# ------------------------------------------------------------------ tiling

def cube_grid(T: int, H: int, W: int) -> tuple[int, int, int]:
    """Cubes along each axis: ceil(T/4), ceil(H/4), ceil(W/4).

    Dataset card, "Shapes": Nq = Nkv = ceil(21/4) ceil(30/4) ceil(52/4) = 624.
    """
    return -(-T // EDGE), -(-H // EDGE), -(-W // EDGE)


def _extent(n: int, i: int) -> int:
    """Tokens of cube i along an axis of n tokens (the last cube may be short)."""
    return min(EDGE, n - EDGE * i)


def cube_sizes(T: int, H: int, W: int) -> np.ndarray:
    """vbs[c]: real (non-pad) tokens in cube c, int32 of shape (Nc,).

    Dataset card, "Shapes" (vbs: real token count per KV cube) and "Operator
    contract" (attend only the first vbs[c] of 64).
    """
    Nt, Nh, Nw = cube_grid(T, H, W)
    vbs = np.empty(Nt * Nh * Nw, dtype=np.int32)
    for ct in range(Nt):
        for ch in range(Nh):
            for cw in range(Nw):
                c = (ct * Nh + ch) * Nw + cw
                vbs[c] = _extent(T, ct) * _extent(H, ch) * _extent(W, cw)
    return vbs


def slot_tokens(T: int, H: int, W: int) -> np.ndarray:
    """Natural token index held by each tiled slot, int64 (Nc, 64); -1 = pad.

    Slot u < vbs[c] of cube (ct, ch, cw) holds the token at offset
    (dt, dh, dw) = row-major position u inside the clipped extent (et, eh, ew);
    its natural index is ((4ct+dt) H + 4ch+dh) W + 4cw+dw.
    """
    Nt, Nh, Nw = cube_grid(T, H, W)
    out = np.full((Nt * Nh * Nw, CUBE), -1, dtype=np.int64)
    for ct in range(Nt):
        et = _extent(T, ct)
        for ch in range(Nh):
            eh = _extent(H, ch)
            for cw in range(Nw):
                ew = _extent(W, cw)
                c = (ct * Nh + ch) * Nw + cw
                u = 0
                for dt in range(et):
                    for dh in range(eh):
                        for dw in range(ew):
                            t, y, x = EDGE * ct + dt, EDGE * ch + dh, EDGE * cw + dw
                            out[c, u] = (t * H + y) * W + x
                            u += 1
    return out


def tile(x_nat: np.ndarray, T: int, H: int, W: int, order=None) -> tuple[np.ndarray, np.ndarray]:
    """Natural order (B, T*H*W, NH, D) -> cube-major (B, Nc*64, NH, D), plus vbs.

    Works on any dtype (bf16 bit patterns are copied, not converted); padding
    slots are zero. With ``order`` (see ``cube_order``) tiled cube p is the
    row-major cube order[p], and vbs follows the same order.
    """
    x_nat = np.asarray(x_nat)
    B, N, NH, D = x_nat.shape
    assert N == T * H * W, (N, T, H, W)
    src = slot_tokens(T, H, W)
    Nc = src.shape[0]
    vbs = cube_sizes(T, H, W)
    if order is not None:
        order = np.asarray(order)
        assert np.array_equal(np.sort(order), np.arange(Nc)), "order is not a permutation"
        src, vbs = src[order], vbs[order]
    out = np.zeros((B, Nc * CUBE, NH, D), dtype=x_nat.dtype)
    flat = src.reshape(-1)
    real = flat >= 0
    out[:, real] = x_nat[:, flat[real]]
    return out, vbs


def untile(y_t: np.ndarray, T: int, H: int, W: int, order=None) -> np.ndarray:
    """Inverse of ``tile`` (for the same ``order``): cube-major (B, Nc*64, NH, D)
    -> natural order.

    Padding slots are dropped (FastVideo STA guide, "Implementation": the tile
    permutation is inverted to restore the sequential order).
    """
    y_t = np.asarray(y_t)
    B, S, NH, D = y_t.shape
    src = slot_tokens(T, H, W)
    assert S == src.shape[0] * CUBE
    if order is not None:
        src = src[np.asarray(order)]
    out = np.empty((B, T * H * W, NH, D), dtype=y_t.dtype)
    flat = src.reshape(-1)
    real = flat >= 0
    out[:, flat[real]] = y_t[:, real]
    return out


def hilbert_index_3d(x0: int, x1: int, x2: int, bits: int) -> int:
    """Index of the point (x0, x1, x2) (each < 2^bits) on the 3D Hilbert curve.

    J. Skilling, "Programming the Hilbert curve" (AIP Conf. Proc. 707, 2004):
    the coordinates are turned into the curve's "transposed" index (undo the
    excess work bit plane by bit plane from the top, Gray-encode, fix the
    parity), whose bits, read plane by plane from the top with x0 first, form
    the index.
    """
    X = [x0, x1, x2]
    q = 1 << (bits - 1)
    while q > 1:
        low = q - 1
        for i in range(3):
            if X[i] & q:
                X[0] ^= low
            else:
                swap = (X[0] ^ X[i]) & low
                X[0] ^= swap
                X[i] ^= swap
        q >>= 1
    X[1] ^= X[0]
    X[2] ^= X[1]
    fix = 0
    q = 1 << (bits - 1)
    while q > 1:
        if X[2] & q:
            fix ^= q - 1
        q >>= 1
    X = [v ^ fix for v in X]
    h = 0
    for plane in range(bits - 1, -1, -1):
        for v in X:
            h = 2 * h + ((v >> plane) & 1)
    return h


def cube_order(T: int, H: int, W: int, kind: str = "hilbert") -> np.ndarray:
    """Cube order table, int32 (Nc,): entry p is the row-major cube id
    (ct*Nh + ch)*Nw + cw placed at tiled position p.

    VSA blog, "Two-Stage Architecture", pre-stage: tokens are reordered along a
    3D space-filling curve. Reading 15: the 4x4x4 cube is the curve's leaf;
    "hilbert" sorts the cubes by their index on the Hilbert curve of the
    smallest power-of-two box holding the cube grid; "row_major" is the
    identity (reading 1).
    """
    Nt, Nh, Nw = cube_grid(T, H, W)
    n = Nt * Nh * Nw
    if kind == "row_major":
        return np.arange(n, dtype=np.int32)
    assert kind == "hilbert", kind
    bits = max(1, math.ceil(math.log2(max(Nt, Nh, Nw))))
    key = [hilbert_index_3d(c // (Nh * Nw), (c // Nw) % Nh, c % Nw, bits) for c in range(n)]
    return np.argsort(np.asarray(key, dtype=np.int64), kind="stable").astype(np.int32)


# ---------------------------------------------------------------- selector

def mean_pool(x_t: np.ndarray, vbs: np.ndarray) -> np.ndarray:
    """Per-cube mean of the real tokens: (B, Nc*64, NH, D) -> (B, NH, Nc, D).

    VSA blog, "Two-Stage Architecture", Stage 1: each cube is mean-pooled into
    one cube-level vector. Reading 4: the mean is over the vbs[c] real tokens.
    """
    x_t = np.asarray(x_t, dtype=np.float64)
    B, S, NH, D = x_t.shape
    Nc = S // CUBE
    out = np.zeros((B, NH, Nc, D), dtype=np.float64)
    for c in range(Nc):
        n = int(vbs[c])
        if n > 0:
            rows = x_t[:, c * CUBE:c * CUBE + n]          # (B, n, NH, D)
            out[:, :, c, :] = rows.sum(axis=1) / n
    return out


def cube_scores(Qc: np.ndarray, Kc: np.ndarray) -> np.ndarray:
    """S[b, h, i, j] = Qc[b, h, i] . Kc[b, h, j] (cube-to-cube scores).

    VSA blog, "Generating Sparsity Patterns": an einsum 'bhqd,bhkd->bhqk' of the
    pooled blocks; Wan 2.2 INT8 blog, "Decoupling Block Selection": S_ij is the
    dot product of the mean-pooled summaries. Reading 5: no scale, no softmax.
    """
    return np.matmul(np.asarray(Qc, np.float64),
                     np.swapaxes(np.asarray(Kc, np.float64), -1, -2))


def topk_select(S: np.ndarray, k: int) -> np.ndarray:
    """Per row of S, the ids of the k largest scores, score-descending.

    VSA blog, "Two-Stage Architecture" (for each query cube keep the Top-K
    key/value cubes with the highest scores) and "Generating Sparsity Patterns"
    (torch.topk over the key axis, whose default order is descending). Reading
    6: equal scores are ordered by ascending cube id. A stable sort of the
    negated scores yields exactly that order.
    """
    S = np.asarray(S, dtype=np.float64)
    n = S.shape[-1]
    assert 1 <= k <= n, (k, n)
    order = np.argsort(-S, axis=-1, kind="stable")
    return np.ascontiguousarray(order[..., :k]).astype(np.int32)


def select(q_t: np.ndarray, k_t: np.ndarray, vbs: np.ndarray, k: int):
    """Coarse stage: mean-pool, cube scores, top-k. Returns (topk_idx, S)."""
    Qc = mean_pool(q_t, vbs)
    Kc = mean_pool(k_t, vbs)
    S = cube_scores(Qc, Kc)
    return topk_select(S, k), S


# --------------------------------------------------------------- fine stage

def cdf_counts(S: np.ndarray, max_k: int, tau: float, scale: float):
    """Wan INT8 blog, "Decoupling Block Selection": sort each row's scores
    (descending, ties by ascending id, as ``topk_select``), take the softmax
    weights w_i = exp((s_i - s_0) * scale) in that order and keep the fewest
    leading cubes whose share of the total weight reaches tau.
    Returns (ids (..., max_k), counts (...)), the counts capped at max_k."""
    assert 0.0 < tau <= 1.0
    order = topk_select(S, S.shape[-1])
    ss = np.take_along_axis(np.asarray(S, np.float64), order.astype(np.int64), axis=-1)
    w = np.exp((ss - ss[..., :1]) * scale)
    c = np.cumsum(w, axis=-1)
    n = np.argmax(c >= tau * c[..., -1:], axis=-1) + 1
    return order[..., :max_k], np.minimum(n, max_k).astype(np.int32)


def select_cdf(q_t: np.ndarray, k_t: np.ndarray, vbs: np.ndarray, max_k: int, tau: float,
               sm_scale: float | None = None):
    """Coarse selector with a cumulative-mass threshold: (ids, counts, S)."""
    D = q_t.shape[-1]
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    S = cube_scores(mean_pool(q_t, vbs), mean_pool(k_t, vbs))
    ids, n = cdf_counts(S, max_k, tau, scale)
    return ids, n, S


def _selected_rows(sel: np.ndarray, vbs: np.ndarray) -> np.ndarray:
    """Tiled row indices of the real tokens of the selected cubes."""
    ids = np.asarray(sel, dtype=np.int64)
    n_kv = vbs.shape[0]
    assert np.all((ids >= 0) & (ids < n_kv)), "topk id out of range"
    assert np.unique(ids).size == ids.size, "duplicate topk id in a row"
    parts = [CUBE * j + np.arange(int(vbs[j]), dtype=np.int64) for j in ids]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def fwd_unit(q_t, k_t, v_t, topk_idx, vbs, b: int, h: int, c: int,
             sm_scale: float | None = None) -> np.ndarray:
    """The 64 output rows of query cube c of (batch b, head h), float64 (64, D).

    Dataset card, "Operator contract": out = softmax((q k_sel^T)/sqrt(D)) v_sel,
    the selected key/value cubes named by topk_idx, attending only the first
    vbs[j] tokens of cube j. The selected real rows are gathered explicitly,
    the row maximum is subtracted before exp (a softmax is invariant to it),
    and the weights are normalised by their sum.
    """
    D = q_t.shape[-1]
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    rows = _selected_rows(topk_idx[b, h, c], np.asarray(vbs))
    q = np.asarray(q_t[b, c * CUBE:(c + 1) * CUBE, h, :], dtype=np.float64)
    if rows.size == 0:
        return np.zeros((CUBE, D), dtype=np.float64)      # reading 10
    K = np.asarray(k_t[b, rows, h, :], dtype=np.float64)  # (n, D)
    V = np.asarray(v_t[b, rows, h, :], dtype=np.float64)
    s = (q @ K.T) * scale                                  # (64, n)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def fwd_units(q_t, k_t, v_t, topk_idx, vbs, units, sm_scale=None) -> np.ndarray:
    """Output rows for a list of (b, h, c) units: float64 (len(units), 64, D)."""
    D = q_t.shape[-1]
    out = np.empty((len(units), CUBE, D), dtype=np.float64)
    for i, (b, h, c) in enumerate(units):
        out[i] = fwd_unit(q_t, k_t, v_t, topk_idx, vbs, b, h, c, sm_scale)
    return out


def fwd(q_t, k_t, v_t, topk_idx, vbs, sm_scale=None) -> np.ndarray:
    """Whole fine stage: (B, Nq*64, NH, D) float64 for every (b, h, c)."""
    B, S, NH, D = q_t.shape
    Nq = S // CUBE
    assert topk_idx.shape[:3] == (B, NH, Nq), topk_idx.shape
    out = np.empty((B, S, NH, D), dtype=np.float64)
    for b in range(B):
        for h in range(NH):
            for c in range(Nq):
                out[b, c * CUBE:(c + 1) * CUBE, h, :] = fwd_unit(
                    q_t, k_t, v_t, topk_idx, vbs, b, h, c, sm_scale)
    return out


def fwd_unit_stats(q_t, k_t, v_t, ids, vbs, b: int, h: int, c: int,
                   sm_scale: float | None = None):
    """Rows of query cube c of (b, h) attending the real tokens of cubes ``ids``:
    (out (64, D), lse (64,), max_prob (64,)), float64.

    VSA blog, "Sparse Traversal": only the listed blocks are visited. Wan INT8
    blog, "Dynamic Sparsity Budgeting via Softmax Normalizer Registers": with
    m_i the row max and l_i = sum_j exp(s_ij - m_i), max_prob_i = 1 / l_i;
    the log-sum-exp of the row is m_i + log l_i.
    """
    D = q_t.shape[-1]
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    rows = _selected_rows(np.asarray(ids), np.asarray(vbs))
    if rows.size == 0:
        return (np.zeros((CUBE, D)), np.full(CUBE, -np.inf), np.zeros(CUBE))
    q = np.asarray(q_t[b, c * CUBE:(c + 1) * CUBE, h, :], dtype=np.float64)
    K = np.asarray(k_t[b, rows, h, :], dtype=np.float64)
    V = np.asarray(v_t[b, rows, h, :], dtype=np.float64)
    s = (q @ K.T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1)
    return (p @ V) / l[:, None], m[:, 0] + np.log(l), 1.0 / l


def fwd_lut(q_t, k_t, v_t, kv_block_idx, valid_block_num, vbs, sm_scale=None):
    """Fine stage driven by a block lookup table: query cube (b, h, c) attends
    the first valid_block_num[b, h, c] ids of kv_block_idx[b, h, c]
    (all of them if valid_block_num is None). Returns out (B, Nq*64, NH, D),
    lse and max_prob (B, NH, Nq*64), float64."""
    B, S, NH, D = q_t.shape
    Nq = S // CUBE
    assert kv_block_idx.shape[:3] == (B, NH, Nq), kv_block_idx.shape
    max_kv = kv_block_idx.shape[3]
    out = np.empty((B, S, NH, D))
    lse = np.empty((B, NH, S))
    mp = np.empty((B, NH, S))
    for b in range(B):
        for h in range(NH):
            for c in range(Nq):
                n = max_kv if valid_block_num is None else int(valid_block_num[b, h, c])
                assert 0 <= n <= max_kv, "valid_block_num outside [0, max_kv]"
                o, e, x = fwd_unit_stats(q_t, k_t, v_t, kv_block_idx[b, h, c, :n], vbs, b, h, c,
                                         sm_scale)
                out[b, c * CUBE:(c + 1) * CUBE, h, :] = o
                lse[b, h, c * CUBE:(c + 1) * CUBE] = e
                mp[b, h, c * CUBE:(c + 1) * CUBE] = x
    return out, lse, mp


# ------------------------------------------------------ coarse output, combine

def coarse_output(q_t, k_t, v_t, vbs, sm_scale=None) -> np.ndarray:
    """Coarse-stage output Oc (B, NH, Nc, D), float64.

    VSA blog, "Two-Stage Architecture": the coarse stage attends among the
    mean-pooled cubes. Per (b, h): Oc = softmax(Qc Kc^T * sm_scale) Vc with Qc,
    Kc, Vc from ``mean_pool``, the softmax over the key cubes with vbs[j] > 0
    (reading 13).
    """
    D = q_t.shape[-1]
    scale = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    vbs = np.asarray(vbs)
    Qc, Kc, Vc = mean_pool(q_t, vbs), mean_pool(k_t, vbs), mean_pool(v_t, vbs)
    real = vbs > 0
    B, NH, Nc, _ = Qc.shape
    out = np.zeros((B, NH, Nc, D))
    if not real.any():
        return out
    for b in range(B):
        for h in range(NH):
            s = (Qc[b, h] @ Kc[b, h][real].T) * scale          # (Nc, n_real)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, h] = (p @ Vc[b, h][real]) / p.sum(axis=1, keepdims=True)
    return out


def gated_combine(o_fine, o_coarse, gate_coarse, gate_fine) -> np.ndarray:
    """out[b, s, h, :] = gate_coarse[b, s, h, :] * Oc[b, h, s // 64, :]
    + gate_fine[b, s, h, :] * o_fine[b, s, h, :], float64 (B, Nc*64, NH, D).

    VSA blog, "Two-Stage Architecture": the final output mixes the coarse-stage
    and fine-stage outputs through gates (reading 14: elementwise tensors).
    """
    o_coarse = np.asarray(o_coarse, np.float64)
    B, NH, Nc, D = o_coarse.shape
    oc_rows = np.repeat(np.transpose(o_coarse, (0, 2, 1, 3)), CUBE, axis=1)  # (B, Nc*64, NH, D)
    return (np.asarray(gate_coarse, np.float64) * oc_rows
            + np.asarray(gate_fine, np.float64) * np.asarray(o_fine, np.float64))


# ------------------------------------------------------------ mask -> LUT

def mask_to_lut(block_mask, max_kv: int):
    """Block relation matrix -> lookup table.

    VSA blog, "Sparse Encoding in CK Tile": Jenga's B[i][j] (attend when
    nonzero) versus VSA's list of selected block ids plus a valid count per
    query block. Per row: the ids j with B[i][j] != 0 in ascending order, the
    first max_kv of them kept; count = min(#set, max_kv). Returns (ids
    (..., max_kv) int32 with -1 past the count, counts (...) int32, number of
    rows with more than max_kv set cells).
    """
    m = np.asarray(block_mask) != 0
    lead = m.shape[:-1]
    ids = np.full(lead + (max_kv,), -1, dtype=np.int32)
    cnt = np.zeros(lead, dtype=np.int32)
    truncated = 0
    for r in np.ndindex(*lead):
        on = np.flatnonzero(m[r])
        truncated += int(on.size > max_kv)
        keep = on[:max_kv]
        ids[r][:keep.size] = keep
        cnt[r] = keep.size
    return ids, cnt, truncated
