"""Helpers shared by the GPU parity tests: uploads, the oracle-side reference
values, and the acceptance rules.

Acceptance rules (Wan2.2 Production Values dataset card, section "Scoring /
loss"): the output is finite everywhere; per-head cosine >= 0.9999 (each head
flattened over (S, D)); max |delta| <= 3e-2; mean |delta| <= 2e-4 (the card's
1e-4 is against a Triton bf16 output; here the reference is the oracle's
float64 result rounded to bf16). Top-k ids must equal the oracle's except for
swaps between cubes whose scores differ by less than 1e-4 relative.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

COS_MIN = 0.9999
MAX_ABS = 3e-2
MEAN_ABS = 2e-4
TOPK_REL = 1e-4
U32 = 2.0 ** -24       # fp32 unit roundoff


def to_gpu_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bfloat16 CUDA tensor (bit-exact)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def from_gpu_bf16(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> uint16 bit patterns on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def gamma(n: int) -> float:
    return n * U32 / (1 - n * U32)


def topk_check(gpu_idx: np.ndarray, ora_idx: np.ndarray, S: np.ndarray,
               Qc: np.ndarray, Kc: np.ndarray, Qa: np.ndarray, Ka: np.ndarray, n_pool: int):
    """Position-wise tie-tolerant comparison of top-k rows.

    S: oracle float64 scores (B, NH, Nq, Nkv); Qc/Kc: oracle float64 means;
    Qa/Ka: means of |x| (the scale of the fp32 pooling error). A GPU id may
    differ from the oracle's at position p only if the two scores agree within
    TOPK_REL relative, widened by the fp32 error bound of the GPU's pooling
    (sum of n_pool terms) and dot product (D terms).
    Returns (ok, n_positions_differing, worst_excess).
    """
    B, NH, Nq, k = ora_idx.shape
    D = Qc.shape[-1]
    assert gpu_idx.shape == ora_idx.shape
    Nkv = S.shape[-1]
    if gpu_idx.min() < 0 or gpu_idx.max() >= Nkv:
        return False, -1, math.inf
    srt = np.sort(gpu_idx, axis=-1)
    if np.any(srt[..., 1:] == srt[..., :-1]):
        return False, -1, math.inf
    diff = gpu_idx != ora_idx
    n_diff = int(diff.sum())
    if n_diff == 0:
        return True, 0, 0.0
    worst = 0.0
    g_pool = gamma(n_pool + 1)
    for b, h, i, p in zip(*np.nonzero(diff)):
        jg, jo = int(gpu_idx[b, h, i, p]), int(ora_idx[b, h, i, p])
        sg, so = S[b, h, i, jg], S[b, h, i, jo]
        eps = 0.0
        for j in (jg, jo):
            e = (gamma(D) * np.dot(np.abs(Qc[b, h, i]), np.abs(Kc[b, h, j]))
                 + g_pool * (np.dot(Qa[b, h, i], np.abs(Kc[b, h, j]))
                             + np.dot(np.abs(Qc[b, h, i]), Ka[b, h, j])))
            eps = max(eps, e)
        allowed = TOPK_REL * max(abs(sg), abs(so)) + 2 * eps
        worst = max(worst, abs(sg - so) / allowed)
    return worst <= 1.0, n_diff, worst


def fine_metrics(gpu_bits: np.ndarray, ref64: np.ndarray) -> dict:
    """Compare GPU bf16 output rows with the oracle's float64 rows.

    gpu_bits, ref64: (..., NH-major last two axes handled by caller) arrays of
    the same shape (N, NH, D) or (units, 64, D) grouped per head by caller.
    """
    g = oracle.decode_bf16(gpu_bits)
    r = oracle.round_to_bf16(ref64)
    d = np.abs(g - r)
    return {
        "finite": bool(np.all(np.isfinite(g))),
        "max_abs": float(d.max()),
        "mean_abs": float(d.mean()),
        "max_abs_unrounded": float(np.abs(g - ref64).max()),
        "mean_abs_unrounded": float(np.abs(g - ref64).mean()),
    }


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = a.reshape(-1).astype(np.float64)
    b = b.reshape(-1).astype(np.float64)
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def assert_fine_ok(gpu_bits_by_head: dict, ref_by_head: dict, label: str) -> dict:
    """gpu_bits_by_head[h] / ref_by_head[h]: rows of head h (any shape ... x D)."""
    g_all = np.concatenate([gpu_bits_by_head[h].reshape(-1) for h in sorted(ref_by_head)])
    r_all = np.concatenate([ref_by_head[h].reshape(-1) for h in sorted(ref_by_head)])
    m = fine_metrics(g_all, r_all)
    rr = oracle.round_to_bf16
    cos = {h: cosine(oracle.decode_bf16(gpu_bits_by_head[h]), rr(ref_by_head[h]))
           for h in ref_by_head}
    m["min_head_cos"] = min(cos.values())
    print(f"[{label}] {m}", flush=True)
    assert m["finite"], label
    assert m["min_head_cos"] >= COS_MIN, (label, m)
    assert m["max_abs"] <= MAX_ABS, (label, m)
    assert m["mean_abs"] <= MEAN_ABS, (label, m)
    return m


def sample_units(vbs: np.ndarray, NH: int, per_head: int, seed: int, extra_heads=()):
    """Seeded query cubes per head: at least 2 from each vbs class, the rest
    uniform; every cube of the heads in extra_heads."""
    rng = np.random.default_rng(seed)
    Nc = vbs.size
    units = []
    classes = np.unique(vbs)
    for h in range(NH):
        if h in extra_heads:
            units += [(0, h, c) for c in range(Nc)]
            continue
        chosen = []
        for v in classes:
            pool = np.nonzero(vbs == v)[0]
            chosen += list(rng.choice(pool, size=min(2, pool.size), replace=False))
        rest = np.setdiff1d(np.arange(Nc), chosen)
        n_more = max(0, min(per_head - len(chosen), rest.size))
        chosen += list(rng.choice(rest, size=n_more, replace=False))
        units += [(0, h, int(c)) for c in sorted(chosen)]
    return units


class ConfigRun:
    """One workload on the device and on the oracle, computed lazily.

    The device tiles the natural-order inputs itself; the oracle tiles its own
    copy. The fine stage on the device is fed the oracle's indices.
    """

    def __init__(self, case):
        import video_dit_block_amd as vsa

        self.case = c = case
        print(f"[{c.name}] B={c.B} grid={c.T}x{c.H}x{c.W} NH={c.NH} D={c.D} topk={c.topk} "
              f"seed={c.seed} outlier_head={c.outlier_head}", flush=True)
        self.vsa = vsa
        self.q_nat, self.k_nat, self.v_nat = (to_gpu_bf16(a) for a in (c.q, c.k, c.v))
        self.qt, self.vbs = vsa.tile(self.q_nat, c.T, c.H, c.W)
        self.kt, _ = vsa.tile(self.k_nat, c.T, c.H, c.W)
        self.vt, _ = vsa.tile(self.v_nat, c.T, c.H, c.W)
        torch.cuda.synchronize()
        self.vbs_o = oracle.cube_sizes(c.T, c.H, c.W)
        self.Nc = self.vbs_o.size
        self._tiled_o = {}
        self._sel = None

    def tiled_oracle(self, name):
        if name not in self._tiled_o:
            self._tiled_o[name] = oracle.tile(getattr(self.case, name), self.case.T,
                                              self.case.H, self.case.W)[0]
        return self._tiled_o[name]

    def head64(self, name, h):
        """Oracle-tiled tensor `name` of head h, float64 (B, S, 1, D)."""
        return oracle.decode_bf16(self.tiled_oracle(name)[:, :, h:h + 1, :])

    def oracle_select(self):
        """Oracle selector, head by head: (idx, S, Qc, Kc, |q| means, |k| means)."""
        if self._sel is None:
            c, Nc = self.case, self.Nc
            shp = (c.B, c.NH, Nc)
            S = np.empty(shp + (Nc,))
            Qc, Kc, Qa, Ka = (np.empty(shp + (c.D,)) for _ in range(4))
            for h in range(c.NH):
                q, k = self.head64("q", h), self.head64("k", h)
                Qc[:, h] = oracle.mean_pool(q, self.vbs_o)[:, 0]
                Kc[:, h] = oracle.mean_pool(k, self.vbs_o)[:, 0]
                Qa[:, h] = oracle.mean_pool(np.abs(q), self.vbs_o)[:, 0]
                Ka[:, h] = oracle.mean_pool(np.abs(k), self.vbs_o)[:, 0]
                S[:, h] = oracle.cube_scores(Qc[:, h:h + 1], Kc[:, h:h + 1])[:, 0]
            idx = oracle.topk_select(S, c.topk)
            self._sel = (idx, S, Qc, Kc, Qa, Ka)
        return self._sel

    def oracle_rows(self, units, idx):
        """Oracle output rows of (b, h, c) units with selection idx: dict h -> (n, 64, D)."""
        by_head = {}
        for b, h, cc in units:
            by_head.setdefault(h, []).append((b, cc))
        out = {}
        for h, lst in by_head.items():
            q, k, v = self.head64("q", h), self.head64("k", h), self.head64("v", h)
            out[h] = np.stack([oracle.fwd_unit(q, k, v, idx[:, h:h + 1], self.vbs_o, b, 0, cc)
                               for b, cc in lst])
        return out

    @staticmethod
    def device_rows(out_bits, units):
        by_head = {}
        for b, h, cc in units:
            by_head.setdefault(h, []).append(out_bits[b, 64 * cc:64 * (cc + 1), h])
        return {h: np.stack(v) for h, v in by_head.items()}


def coarse_tolerance(Qc, Kc, Vc, Qa, Ka, Va, vbs, scale, n_pool: int = 64):
    """Per (i, d) bound on |device o_coarse - oracle| for one (b, h), from the
    kernels' fp32 arithmetic (u = 2^-24):
    * pooled means are off by <= gamma_{n+1} times the mean of |x|;
    * score S_ij = Qc_i . Kc_j is then off by <= e_ij = gamma_D |Qc_i|.|Kc_j|
      + gamma_{n+1} (Qa_i.|Kc_j| + |Qc_i|.Ka_j); e_i = max over real j;
    * weight exp2((S_ij - m_i) scale log2 e): relative error <= delta_i =
      (2 e_i + 6 u max_j |S_ij|) scale + 2^-22 (argument roundings, the
      hardware exp2);
    * normalisation and the Nc-term fp32 sums add (2 Nc + 4) u relative;
    so |dO_id| <= (2 delta_i + (2 Nc + 4) u) max_j |Vc_jd| + gamma_{n+1}
    max_j Va_jd. Qc.. are (Nc, D) float64; the maxima run over key cubes with
    vbs > 0."""
    real = np.asarray(vbs) > 0
    Nc, D = Qc.shape
    aQ, aK = np.abs(Qc), np.abs(Kc)
    g = gamma(n_pool + 1)
    e = gamma(D) * aQ @ aK.T + g * (Qa @ aK.T + aQ @ Ka.T)
    e_i = e[:, real].max(axis=1)
    smax = np.abs(Qc @ Kc.T)[:, real].max(axis=1)
    delta = (2 * e_i + 6 * U32 * smax) * scale + 2.0 ** -22
    vmax = np.abs(Vc[real]).max(axis=0)
    return (2 * delta + (2 * Nc + 4) * U32)[:, None] * vmax[None, :] + g * Va[real].max(axis=0)[None, :]


def check_coarse(oc_gpu: np.ndarray, head64, vbs, NH: int, sm_scale, label: str) -> float:
    """Every element of o_coarse (B, NH, Nc, D) against the oracle. head64(name,
    h) returns the tiled float64 tensor `name` of head h as (B, S, 1, D).
    Returns the worst error / bound ratio."""
    B, _, Nc, D = oc_gpu.shape
    scale = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    worst = max_err = 0.0
    for h in range(NH):
        q, k, v = head64("q", h), head64("k", h), head64("v", h)
        ref = oracle.coarse_output(q, k, v, vbs, sm_scale)[:, 0]
        pools = [oracle.mean_pool(x, vbs)[:, 0] for x in (q, k, v, np.abs(q), np.abs(k), np.abs(v))]
        for b in range(B):
            tol = coarse_tolerance(*(p[b] for p in pools), vbs, scale)
            d = np.abs(oc_gpu[b, h].astype(np.float64) - ref[b])
            assert np.all(np.isfinite(oc_gpu[b, h])), (label, b, h)
            ratio = float(np.max(d / np.maximum(tol, 1e-300)))
            worst, max_err = max(worst, ratio), max(max_err, float(d.max()))
            assert ratio <= 1.0, (label, b, h, ratio, float(d.max()))
    print(f"[{label}] o_coarse max |d| {max_err:.3g}, worst |d| / bound {worst:.3g}", flush=True)
    return worst


def combine_check(out_bits, o_fine_bits, o_coarse, gc_bits, gf_bits, label: str) -> None:
    """Gated combine against the oracle: |out - exact| <= 1/2 ulp_bf16(exact)
    + 2^-23 (|g_c o_c| + |g_f o_f|) (fp32 product and fma, then bf16 rounding
    to nearest even)."""
    of, gc, gf = (oracle.decode_bf16(x) for x in (o_fine_bits, gc_bits, gf_bits))
    oc = np.asarray(o_coarse, np.float64)
    exact = oracle.gated_combine(of, oc, gc, gf)
    oc_rows = np.repeat(np.transpose(oc, (0, 2, 1, 3)), 64, axis=1)
    err32 = 2.0 ** -23 * (np.abs(gc * oc_rows) + np.abs(gf * of))
    mag = np.abs(exact) + err32
    ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 2.0 ** -126))) - 7)
    got = oracle.decode_bf16(out_bits)
    d = np.abs(got - exact)
    ratio = d / (0.5 * ulp + err32)
    n_eq = int(np.sum(got == oracle.round_to_bf16(exact)))
    print(f"[{label}] equal to the rounded exact value: {n_eq}/{got.size}; worst |d| / bound "
          f"{ratio.max():.6f}", flush=True)
    assert np.all(ratio <= 1.0), label


def stat_tolerance_rows(q_rows, k_all, ids, vbs, scale):
    """Per query row, the bound on |d lse| of the fine kernel (and on the
    relative error of max_prob, halved): l is the fp32 sum of fp16-rounded
    weights (2^-11 + n 2^-24 relative), and each score is an fp32 MFMA dot
    product of bf16 inputs (|d s| <= gamma_D sum_d |q_d k_d|, Higham), which
    moves lse by at most twice that times sm_scale. q_rows (64, D) and k_all
    (S, D) are float64 tiled rows of one (b, h)."""
    rows = np.concatenate([64 * j + np.arange(vbs[j]) for j in ids]) if len(ids) else np.zeros(0, int)
    if rows.size == 0:
        return np.zeros(q_rows.shape[0])
    D = q_rows.shape[-1]
    a = np.abs(q_rows) @ np.abs(k_all[rows]).T
    return 2.0 ** -11 + rows.size * 2.0 ** -24 + 2 * gamma(D) * scale * a.max(axis=1)
