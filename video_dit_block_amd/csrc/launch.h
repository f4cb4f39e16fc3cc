// Internal launch functions of libvsa (host side). The C ABI in api.hip
// validates arguments and then calls these; each enqueues its kernels on
// `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vsa {

// order == nullptr: row-major cube order; else tiled cube p is row-major
// cube order[p].
hipError_t launch_tile(const uint16_t* x, uint16_t* x_tiled, int32_t* vbs,
                       const int32_t* order, int B, int T, int H, int W, int NH, int D,
                       hipStream_t stream);
hipError_t launch_untile(const uint16_t* y_tiled, uint16_t* y, const int32_t* order, int B,
                         int T, int H, int W, int NH, int D, hipStream_t stream);
// Host: the cube order table (kind 0 row-major, 1 Hilbert); false if the
// grid is too large for a 63-bit Hilbert index.
bool cube_order(int T, int H, int W, int kind, int32_t* order);
// Block mask [rows][Nkv] (nonzero = attend) -> ascending ids per row, count
// per row (capped at max_kv); rows over the cap add 1 to *n_truncated.
hipError_t launch_mask_to_lut(const uint8_t* mask, int64_t rows, int Nkv, int max_kv,
                              int32_t* kv_block_idx, int32_t* valid_block_num,
                              int32_t* n_truncated, hipStream_t stream);

// Workspace carve-up of vsa_select: pooled q, pooled k, scores.
struct SelectWorkspace {
  size_t qc_off, kc_off, s_off, total;
};
SelectWorkspace select_workspace(int B, int NH, int Nc, int D);

// Selector pieces: mean of the real rows of every cube into fp32
// [B][NH][Nc][D] (launch_pool: one tensor into xc; launch_pool_scores: q and k
// into the workspace's Qc and Kc, then S = Qc . Kc^T), and the per-row top-k
// (with the CDF count when valid != nullptr) over S [BH][Nc][Nc]. row_nh > 0:
// the tiled rows hold row_nh heads, of which the NH from the given pointers
// on are pooled (0 = NH).
hipError_t launch_pool(const uint16_t* x_tiled, const int32_t* vbs, int B, int Nc, int NH,
                       int D, float* xc, hipStream_t stream);
hipError_t launch_pool_scores(const uint16_t* q_tiled, const uint16_t* k_tiled,
                              const int32_t* vbs, int B, int Nc, int NH, int D,
                              void* workspace, hipStream_t stream, int row_nh = 0);
hipError_t launch_topk(const float* s, int BH, int Nc, int topk, int32_t* topk_idx,
                       int32_t* valid, float scale, float tau, hipStream_t stream);

// Coarse stage: its workspace is the selector's (Qc, Kc, S) followed by Vc.
// Pools q, k and v, scores the cubes, optionally writes the top-k ids
// (topk_idx != nullptr), and writes O_c = softmax(S scale) V_c over the key
// cubes holding a real token, fp32 [B][NH][Nc][D].
size_t coarse_workspace_bytes(int B, int NH, int Nc, int D);
hipError_t launch_coarse(const uint16_t* q_tiled, const uint16_t* k_tiled,
                         const uint16_t* v_tiled, const int32_t* vbs, int B, int Nc, int NH,
                         int D, int topk, int32_t* topk_idx, float scale, float* o_coarse,
                         void* workspace, hipStream_t stream);
// out = gate_c * O_c[cube of the row] + gate_f * o_fine, rounded to bf16.
hipError_t launch_gate_combine(const uint16_t* o_fine, const float* o_coarse,
                               const uint16_t* gate_c, const uint16_t* gate_f, uint16_t* out,
                               int B, int Nc, int NH, int D, hipStream_t stream);

// valid != nullptr: also write the CDF count per row (scale, tau). row_nh as
// for launch_pool_scores.
hipError_t launch_select(const uint16_t* q_tiled, const uint16_t* k_tiled,
                         const int32_t* vbs, int B, int Nc, int NH, int D,
                         int topk, int32_t* topk_idx, int32_t* valid, float scale, float tau,
                         void* workspace, hipStream_t stream, int row_nh = 0);

// Key-range splits of the fine stage: at most kMaxSplits; fwd_splits gives
// the number used (forced: 0 = chosen from the sizes, 1 = none, 2.. = that
// many; rows of more than 1024 ids are never split).
constexpr int kMaxSplits = 16;
int fwd_splits(int Nkv, int D, int topk, int forced);

// Workspace carve-up of vsa_fwd: an fp16 copy of v in the tiled layout, the
// tile lists of the units ([B*NH*Nq][list_stride] pairs of uint32 quarters),
// the first tile of every split of a unit ([B*NH*Nq][splits + 1]), the
// dispatch order, each unit's dispatch rank and the order's sort keys, the
// per-(workgroup, head) maxima of |v|, the per-(b, h) exponent of v's fp16
// copy, and with splits the partial results: O as fp32
// [B*NH*Nq*splits][64][D] and (m, l, row max, 0) as float4
// [B*NH*Nq*splits][64].
struct FwdWorkspace {
  size_t v16_off, list_off, sbeg_off, order_off, rank_off, key_off, vmax_off, vexp_off,
      part_off, pstat_off, total;
  int list_stride, splits;
};
FwdWorkspace fwd_workspace(int B, int Nq, int Nkv, int NH, int D, int topk, int forced = 0);
// topk_idx rows hold `topk` ids; valid (may be NULL = all) gives the count
// used per row; lse and max_prob (may be NULL) receive per-row statistics.
hipError_t launch_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* topk_idx, const int32_t* valid, const int32_t* vbs,
                      uint16_t* out, float* lse, float* max_prob, int B, int Nq, int Nkv,
                      int NH, int D, int topk, float sm_scale, int forced_splits,
                      void* workspace, hipStream_t stream);

hipError_t launch_validate_topk(const int32_t* topk_idx, int B, int NH, int Nq,
                                int Nkv, int topk, int32_t* bad_count,
                                hipStream_t stream);

}  // namespace vsa
