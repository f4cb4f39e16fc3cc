/*
 * vsa.h -- C ABI of libvsa, the MI355X (gfx950) Video Sparse Attention hot path.
 *
 * The path has three stages:
 *   1. vsa_tile    cube tiling of the (T, H, W) latent grid into 64-token
 *                  4x4x4 cubes (cube-major, padded);
 *   2. vsa_select  the coarse selector: mean-pool q and k per cube, score cube
 *                  against cube, keep the top-k key cubes of every query cube;
 *   3. vsa_fwd     the fine non-causal block-sparse attention over the selected
 *                  cubes.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers to dense row-major buffers that the
 *   caller allocates and owns. The library never allocates, frees or keeps a
 *   pointer past the call.
 * - bf16 tensors are passed as raw 16-bit patterns (vsa_bf16_t).
 * - q, k, v and out are BSHD: [B][S][NH][D], S = tokens (natural order) or
 *   Nc*64 (tiled order). D is 64 or 128.
 * - Every launch is asynchronous on `stream` (a hipStream_t; NULL = the
 *   default stream). Results are ready when that stream reaches the call.
 * - Arguments are validated on the host before anything is launched. A
 *   failed check returns an error status and launches nothing. A failed
 *   launch returns VSA_ERR_HIP. vsa_last_error() describes the last error of
 *   the calling thread.
 * - No function holds state between calls; concurrent calls on different
 *   streams with disjoint outputs are safe.
 *
 * Cube numbering: Nt = ceil(T/4), Nh = ceil(H/4), Nw = ceil(W/4), Nc = Nt*Nh*Nw;
 * cube (ct, ch, cw) has id c = (ct*Nh + ch)*Nw + cw and holds the tokens
 * t in [4ct, 4ct+et), y in [4ch, 4ch+eh), x in [4cw, 4cw+ew) with
 * et = min(4, T-4ct) etc.; vbs[c] = et*eh*ew real tokens occupy slots
 * 0..vbs[c]-1 of the cube in row-major (t, y, x) order; slots vbs[c]..63 are
 * padding.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VSA_ABI_VERSION 6
#define VSA_CUBE 64

typedef uint16_t vsa_bf16_t; /* raw bf16 bits */
typedef void* vsa_stream_t;  /* hipStream_t; NULL = default stream */

typedef enum {
  VSA_OK = 0,
  VSA_ERR_NULL = 1,        /* a required pointer is NULL */
  VSA_ERR_SHAPE = 2,       /* a size is <= 0, inconsistent, or overflows */
  VSA_ERR_UNSUPPORTED = 3, /* D not in {64, 128}, or Nc above VSA_MAX_CUBES */
  VSA_ERR_RANGE = 4,       /* topk outside [1, Nkv] */
  VSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  VSA_ERR_HIP = 6          /* no device, or the HIP runtime reported an error */
} vsa_status;

/* Largest cube count vsa_select accepts (its per-row sort holds one key per
 * cube in LDS). */
#define VSA_MAX_CUBES 8192

/* ABI version of the loaded library (VSA_ABI_VERSION it was built with). */
int32_t vsa_abi_version(void);

/* Static string naming a status code; never NULL. */
const char* vsa_status_string(int32_t status);

/* Message describing the last error returned on the calling thread ("" if
 * none). Valid until the next libvsa call on this thread. */
const char* vsa_last_error(void);

/* Host, pure. Number of 4x4x4 cubes of a T x H x W grid: ceil(T/4) ceil(H/4)
 * ceil(W/4) (Wan2.2 Production Values dataset card, section "Shapes":
 * 624 = 6 x 8 x 13 for 21 x 30 x 52). Returns -1 if a size is <= 0. */
int32_t vsa_num_cubes(int32_t T, int32_t H, int32_t W);

/* Host, pure. Writes vbs[c] = real tokens of cube c for c < vsa_num_cubes()
 * into the HOST buffer vbs of n_vbs entries (dataset card, "Shapes": vbs is the
 * real, non-pad token count per KV cube). Errors: VSA_ERR_NULL, VSA_ERR_SHAPE
 * (bad grid or n_vbs too small). */
int32_t vsa_vbs_host(int32_t T, int32_t H, int32_t W, int32_t* vbs, int32_t n_vbs);

/* Cube tiling (VSA: Accelerating Video Diffusion Inference with Sparse
 * Attention on AMD GPUs, section "Two-Stage Architecture", Stage 1: tokens are
 * grouped into (4, 4, 4) cubes of 64 tokens; dataset card, "Shapes": the
 * sequence is cube-major and padded, S_padded = Nc x 64).
 *   x        [B][T*H*W][NH][D] bf16, natural row-major (t, y, x) token order
 *   x_tiled  [B][Nc*64][NH][D] bf16 output; padding slots are written as 0
 *   vbs      [Nc] int32 device output, or NULL to skip
 * x and x_tiled must not overlap. Errors: VSA_ERR_NULL, VSA_ERR_SHAPE,
 * VSA_ERR_UNSUPPORTED, VSA_ERR_HIP. */
int32_t vsa_tile(const vsa_bf16_t* x, vsa_bf16_t* x_tiled, int32_t* vbs,
                 int32_t B, int32_t T, int32_t H, int32_t W, int32_t NH,
                 int32_t D, vsa_stream_t stream);

/* Inverse of vsa_tile: drops the padding slots (FastVideo Sliding Tile
 * Attention guide, section "Implementation": the tile permutation is inverted
 * to restore the sequential video order).
 *   y_tiled  [B][Nc*64][NH][D] bf16;  y  [B][T*H*W][NH][D] bf16 output.
 * Errors as vsa_tile. */
int32_t vsa_untile(const vsa_bf16_t* y_tiled, vsa_bf16_t* y, int32_t B,
                   int32_t T, int32_t H, int32_t W, int32_t NH, int32_t D,
                   vsa_stream_t stream);

/* Cube orders for vsa_tile_ordered (VSA blog, "Two-Stage Architecture",
 * pre-stage: tokens are reordered along a 3D space-filling curve so that each
 * attention block covers a compact spatial-temporal region; the curve is not
 * named). */
#define VSA_ORDER_ROW_MAJOR 0 /* tiled cube p = row-major cube p (vsa_tile's order) */
#define VSA_ORDER_HILBERT 1   /* 3D Hilbert curve over the cube grid */

/* Host, pure. Writes order[p] = the row-major id (ct * Nh + ch) * Nw + cw of the
 * cube placed at tiled position p, for p < vsa_num_cubes(T, H, W), into the
 * HOST buffer order of n_order entries. VSA_ORDER_HILBERT sorts the cubes by
 * their index on the 3D Hilbert curve of the smallest power-of-two box that
 * holds the cube grid (J. Skilling, "Programming the Hilbert curve", AIP Conf.
 * Proc. 707, 2004: axes-to-transpose transform, bits interleaved with ct
 * first), so consecutive cubes of a power-of-two grid are face neighbours.
 * Errors: VSA_ERR_NULL, VSA_ERR_SHAPE (bad grid, n_order too small),
 * VSA_ERR_RANGE (kind), VSA_ERR_UNSUPPORTED (a grid side above 2^21 cubes). */
int32_t vsa_cube_order_host(int32_t T, int32_t H, int32_t W, int32_t kind, int32_t* order,
                            int32_t n_order);

/* vsa_tile with a cube order: tiled cube p holds row-major cube order[p], and
 * vbs[p] is that cube's real-token count. order is a DEVICE array of
 * vsa_num_cubes(T, H, W) int32 forming a permutation (a precondition; entries
 * are clamped into range, so a bad table gives wrong rows but no access out
 * of bounds). The selector and the fine stage take the result as they take
 * vsa_tile's. Other arguments and errors as vsa_tile (VSA_ERR_NULL also for a
 * NULL order). */
int32_t vsa_tile_ordered(const vsa_bf16_t* x, vsa_bf16_t* x_tiled, int32_t* vbs,
                         const int32_t* order, int32_t B, int32_t T, int32_t H, int32_t W,
                         int32_t NH, int32_t D, vsa_stream_t stream);

/* Inverse of vsa_tile_ordered for the same order table. Errors as
 * vsa_untile (VSA_ERR_NULL also for a NULL order). */
int32_t vsa_untile_ordered(const vsa_bf16_t* y_tiled, vsa_bf16_t* y, const int32_t* order,
                           int32_t B, int32_t T, int32_t H, int32_t W, int32_t NH, int32_t D,
                           vsa_stream_t stream);

/* Bytes of device workspace vsa_select needs: pooled q and k (fp32,
 * [B][NH][Nc][D] each) and the cube score matrix (fp32, [B][NH][Nc][Nc]).
 * Returns 0 for invalid sizes. */
size_t vsa_select_workspace_bytes(int32_t B, int32_t NH, int32_t Nc, int32_t D);

/* Coarse selector (VSA blog, "Two-Stage Architecture", Stage 1, and section
 * "Generating Sparsity Patterns"; Optimizing block-sparse INT8 attention and
 * multi-expert step caching for Wan 2.2, section "Decoupling Block Selection
 * from Sparse CUDA Kernels"):
 *   Qc[b,h,c] = mean of q_tiled[b, 64c+u, h, :] over u < vbs[c]   (fp32)
 *   Kc likewise from k_tiled
 *   S[b,h,i,j] = Qc[b,h,i] . Kc[b,h,j]                           (fp32)
 *   topk_idx[b,h,i,:] = ids of the topk largest S[b,h,i,:], score
 *                       descending, equal scores by ascending id.
 *   q_tiled, k_tiled  [B][Nc*64][NH][D] bf16 (padding values are ignored)
 *   vbs               [Nc] int32 device, each in [1, 64]
 *   topk_idx          [B][NH][Nc][topk] int32 device output
 *   workspace         device buffer of >= vsa_select_workspace_bytes() bytes,
 *                     256-byte aligned; contents on return are unspecified.
 * Errors: VSA_ERR_NULL, VSA_ERR_SHAPE, VSA_ERR_UNSUPPORTED, VSA_ERR_RANGE,
 * VSA_ERR_WORKSPACE, VSA_ERR_HIP. */
int32_t vsa_select(const vsa_bf16_t* q_tiled, const vsa_bf16_t* k_tiled,
                   const int32_t* vbs, int32_t B, int32_t Nc, int32_t NH,
                   int32_t D, int32_t topk, int32_t* topk_idx, void* workspace,
                   size_t workspace_bytes, vsa_stream_t stream);

/* vsa_select without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Computes exactly what vsa_select computes, with the
 * same kernels, into topk_idx; its scratch (pooled q and k, the cube scores)
 * is a device array of vsa_select_noalloc_max_bytes() = 64 MiB inside the
 * library, one per GPU, held from its first use on that GPU until the process
 * ends. The (batch, head) pairs are processed in chunks of as many heads as
 * fit (30 at the Wan shape, 4 at Nc = 1920), all on `stream`. Nothing in the
 * scratch needs clearing: every byte a call reads it has written first.
 * Every call on one GPU shares that GPU's scratch and leaves its contents
 * behind: calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race and give undefined ids; order
 * them on one stream. No device memory is allocated or freed. Errors: as for
 * vsa_select, without VSA_ERR_WORKSPACE; VSA_ERR_UNSUPPORTED also when one
 * head's workspace (vsa_select_workspace_bytes(1, 1, Nc, D)) exceeds the
 * scratch (Nc above about 4000 at D = 128). */
size_t vsa_select_noalloc_max_bytes(void);
int32_t vsa_select_noalloc(const vsa_bf16_t* q_tiled, const vsa_bf16_t* k_tiled,
                           const int32_t* vbs, int32_t B, int32_t Nc, int32_t NH, int32_t D,
                           int32_t topk, int32_t* topk_idx, vsa_stream_t stream);

/* Coarse selector with a cumulative-mass threshold (Optimizing block-sparse
 * INT8 attention and multi-expert step caching for Wan 2.2, section
 * "Decoupling Block Selection from Sparse CUDA Kernels": sort the block scores
 * of each query block and keep key blocks by a cumulative distribution
 * threshold). Scores S as for vsa_select; per row, with the scores sorted
 * descending (equal scores by ascending id) as s_0 >= s_1 >= ... and
 * w_i = exp((s_i - s_0) * sm_scale), Z = sum over all Nc cubes of w_i:
 *   kv_block_idx[b,h,i,:]   the max_k leading ids of that order (the
 *                           vsa_select result for topk = max_k)
 *   valid_block_num[b,h,i]  the smallest n >= 1 with w_0 + ... + w_{n-1}
 *                           >= tau * Z, capped at max_k
 * The pair is the lookup table vsa_fwd_lut takes. The sums run in fp32 (a
 * count can differ from an exact one where the cumulative mass is within
 * fp32 rounding of tau * Z).
 *   max_k            in [1, Nc]
 *   tau              in (0, 1]
 *   sm_scale         softmax scale of the scores; <= 0 selects 1/sqrt(D)
 *   kv_block_idx     [B][NH][Nc][max_k] int32 device output
 *   valid_block_num  [B][NH][Nc] int32 device output
 * Other arguments and the workspace as for vsa_select. Errors: as for
 * vsa_select. */
int32_t vsa_select_cdf(const vsa_bf16_t* q_tiled, const vsa_bf16_t* k_tiled,
                       const int32_t* vbs, int32_t B, int32_t Nc, int32_t NH, int32_t D,
                       int32_t max_k, float tau, float sm_scale, int32_t* kv_block_idx,
                       int32_t* valid_block_num, void* workspace, size_t workspace_bytes,
                       vsa_stream_t stream);

/* Number of key-range splits S the fine stage uses for these sizes
 * (split-KV): each (b, h, query cube) is computed as S items, item s over the
 * selected cubes j with j * S / Nkv == s, run split-major inside each head so
 * that the items resident at once share one key range of the head; a merge
 * pass combines their partial softmax states (the result is that of the
 * unsplit stage up to fp32 rounding order). kv_splits: 0 chooses (S > 1 only
 * once one head's K plus its fp16 V copy, Nkv * 64 * D * 4 bytes, exceeds
 * 32 MiB: about 32 MiB of them per split, at least 8 selected cubes per split
 * on average, at most 16), 1 turns splitting off, 2..16 asks for that many.
 * Rows of more than 1024 ids are never split. Returns 0 for invalid
 * arguments (kv_splits outside [0, 16], topk outside [1, Nkv]). Host-only. */
int32_t vsa_fwd_splits(int32_t Nkv, int32_t D, int32_t topk, int32_t kv_splits);

/* Bytes of device workspace vsa_fwd needs for these sizes: an fp16 copy of v
 * in the tiled layout (B * Nkv * 64 * NH * D * 2 bytes), then, per (b, h,
 * query cube) (B * NH * Nq of them), the list of the 32-row tiles that hold
 * real tokens of its selected cubes ((2 * topk + 4 + (S > 1 ? S : 0))
 * entries of two uint32), the first tile of each split and the tile count
 * (S + 1 int32), the cube at each dispatch position and each cube's dispatch
 * position (one int32 each) and the positions' sort key (two int32); then the largest |v| of every (v pre-pass workgroup, head)
 * (B * Nkv * 8 * NH float32), the per-(b, h) exponent of the fp16 copy
 * (B * NH int32) and, with S > 1 splits (vsa_fwd_splits), the partial
 * results (B * NH * Nq * S * 64 * (D + 4) float32), each part 256-byte
 * aligned. Returns 0 for invalid sizes. The _ex form takes kv_splits as
 * vsa_fwd_splits does; the plain form is kv_splits = 0. */
size_t vsa_fwd_workspace_bytes(int32_t B, int32_t Nq, int32_t Nkv, int32_t NH,
                               int32_t D, int32_t topk);
size_t vsa_fwd_workspace_bytes_ex(int32_t B, int32_t Nq, int32_t Nkv, int32_t NH,
                                  int32_t D, int32_t topk, int32_t kv_splits);

/* Fine stage: non-causal block-sparse attention (Wan2.2 Production Values
 * dataset card, section "Operator contract"; VSA blog, "Two-Stage
 * Architecture", Stage 2, and "Sparse Traversal"). For every (b, h, query
 * cube c) and each of its 64 rows r (padding rows included):
 *   out[b, 64c+r, h, :] = softmax(q . K^T * sm_scale) . V
 * where K, V are the rows 64j + u, u < vbs[j], of every j in
 * topk_idx[b, h, c, :]. q.k^T runs on bf16 inputs with fp32 accumulation;
 * the softmax is computed online in fp32 with a running row maximum
 * subtracted; the weights (rounded to fp16) and V enter the P.V product as
 * fp16 with fp32 accumulation. V's fp16 copy is exact over the whole bf16
 * range: a head (b, h) whose largest |v| lies outside [2^-4, 65504] is
 * stored scaled by a power of two 2^-e (its largest |v| then in [2^14, 2^15),
 * e in [-90, 113]) and its output multiplied back by 2^e; values below 2^-14
 * (times 2^e) become fp16 subnormals, an absolute error under 2^-24 (times
 * 2^e), at most 2^-20 of the head's largest |v|. The output is rounded to
 * bf16 (nearest even). A row with no real key outputs 0. Large heads run
 * in key-range splits (vsa_fwd_splits with kv_splits = 0).
 *   q         [B][Nq*64][NH][D] bf16, tiled order (padding rows are computed
 *             like real rows)
 *   k, v      [B][Nkv*64][NH][D] bf16, tiled order (padding values ignored)
 *   topk_idx  [B][NH][Nq][topk] int32; every id in [0, Nkv), distinct per row
 *             (a precondition; vsa_validate_topk checks it)
 *   vbs       [Nkv] int32, each in [0, 64]
 *   out       [B][Nq*64][NH][D] bf16 output; must not overlap the inputs
 *   sm_scale  softmax scale; <= 0 selects 1/sqrt(D); must be finite
 *   workspace device buffer of >= vsa_fwd_workspace_bytes(B, Nq, Nkv, NH, D,
 *             topk) bytes, 256-byte aligned, not overlapping the tensors;
 *             contents on return are unspecified (it holds the fp16 copy of v
 *             and the tile lists). The workspace is an addition to the
 *             operator contract's (q, k, v, topk_idx, vbs) -> out: PyTorch
 *             (the caller) owns every allocation, so the fp16 copy of v and
 *             the per-unit lists live in caller memory
 * In the dataset card's self-attention Nq = Nkv; other Nkv are accepted as long
 * as one batch of k spans less than 4 GiB, Nkv * 64 * NH * D * 2 < 2^32
 * (VSA_ERR_UNSUPPORTED beyond).
 * All tensor pointers must be 16-byte aligned. Errors: VSA_ERR_NULL,
 * VSA_ERR_SHAPE, VSA_ERR_UNSUPPORTED, VSA_ERR_RANGE, VSA_ERR_WORKSPACE,
 * VSA_ERR_HIP. */
int32_t vsa_fwd(const vsa_bf16_t* q, const vsa_bf16_t* k, const vsa_bf16_t* v,
                const int32_t* topk_idx, const int32_t* vbs, vsa_bf16_t* out,
                int32_t B, int32_t Nq, int32_t Nkv, int32_t NH, int32_t D,
                int32_t topk, float sm_scale, void* workspace,
                size_t workspace_bytes, vsa_stream_t stream);

/* Fine stage driven by a lookup table with a per-row block count, plus
 * optional per-row softmax statistics. VSA blog, "Block-Sparse Encoding"
 * (kv_block_idx with valid_block_num, the number of valid blocks per query
 * row) and "Sparse Traversal" (the kernel visits the first valid_block_num
 * entries of its row); Wan INT8 blog, "Dynamic Sparsity Budgeting via Softmax
 * Normalizer Registers" (max_prob = 1 / l, l = sum_j exp(s_j - max_j s_j)).
 * Computes what vsa_fwd computes for a row of the first
 * valid_block_num[b][h][c] ids of kv_block_idx[b][h][c][0 .. max_kv); the
 * other entries of the row are not read.
 *   kv_block_idx    [B][NH][Nq][max_kv] int32; the used entries are distinct
 *                   ids in [0, Nkv) (a precondition, as for vsa_fwd)
 *   valid_block_num [B][NH][Nq] int32 device array, each in [0, max_kv]
 *                   (values outside are clamped); NULL means max_kv for every
 *                   row. A count of 0 gives zero output rows.
 *   lse             [B][NH][Nq*64] float32 device array or NULL: per query row,
 *                   the natural-log log-sum-exp of its scaled scores over the
 *                   real keys it attends, log sum_j exp(sm_scale q.k_j); -inf
 *                   for a row without keys
 *   max_prob        [B][NH][Nq*64] float32 device array or NULL: per query
 *                   row, its largest softmax weight 1 / sum_j exp(sm_scale
 *                   (q.k_j - max_i q.k_i)); 0 for a row without keys
 * The workspace is vsa_fwd_workspace_bytes(B, Nq, Nkv, NH, D, max_kv) bytes.
 * lse and max_prob must be 4-byte aligned; every other argument is as for
 * vsa_fwd. The statistics come from the same fp32 running max and the sum of
 * the same fp16-rounded weights that normalise the output. Errors: as for
 * vsa_fwd. */
int32_t vsa_fwd_lut(const vsa_bf16_t* q, const vsa_bf16_t* k, const vsa_bf16_t* v,
                    const int32_t* kv_block_idx, const int32_t* valid_block_num,
                    const int32_t* vbs, vsa_bf16_t* out, float* lse, float* max_prob,
                    int32_t B, int32_t Nq, int32_t Nkv, int32_t NH, int32_t D,
                    int32_t max_kv, float sm_scale, void* workspace,
                    size_t workspace_bytes, vsa_stream_t stream);

/* vsa_fwd_lut with the number of key-range splits chosen by the caller
 * (kv_splits as for vsa_fwd_splits: 0 = chosen from the sizes, as
 * vsa_fwd_lut does; 1 = none; 2..16). The workspace is
 * vsa_fwd_workspace_bytes_ex(B, Nq, Nkv, NH, D, max_kv, kv_splits) bytes.
 * Errors: as for vsa_fwd_lut, and VSA_ERR_RANGE for kv_splits outside
 * [0, 16]. */
int32_t vsa_fwd_lut_ex(const vsa_bf16_t* q, const vsa_bf16_t* k, const vsa_bf16_t* v,
                       const int32_t* kv_block_idx, const int32_t* valid_block_num,
                       const int32_t* vbs, vsa_bf16_t* out, float* lse, float* max_prob,
                       int32_t B, int32_t Nq, int32_t Nkv, int32_t NH, int32_t D,
                       int32_t max_kv, float sm_scale, int32_t kv_splits, void* workspace,
                       size_t workspace_bytes, vsa_stream_t stream);

/* Bytes of device workspace vsa_coarse needs: the vsa_select workspace
 * (pooled q and k, the scores) followed by the pooled v (B * NH * Nc * D
 * float32), each part 256-byte aligned. Returns 0 for invalid sizes. */
size_t vsa_coarse_workspace_bytes(int32_t B, int32_t NH, int32_t Nc, int32_t D);

/* Coarse stage: attention among mean-pooled cubes, and optionally the top-k
 * selection from the same scores. VSA blog, "Two-Stage Architecture": Stage 1
 * pools each cube, scores cube against cube and keeps the Top-K key cubes per
 * query cube; the final output also uses the coarse stage's own output.
 * For each (b, h), with Qc, Kc, Vc the means over the real rows of each cube
 * of q_tiled, k_tiled, v_tiled (as in vsa_select) and S = Qc . Kc^T:
 *   o_coarse[b][h][i][:] = sum_j softmax_j(S[i][j] * sm_scale) Vc[j][:]
 * with j over the key cubes whose vbs[j] > 0 (all weights are 0, and the row
 * is 0, when there is none). Everything runs in fp32.
 *   q_tiled, k_tiled, v_tiled  [B][Nc*64][NH][D] bf16, tiled order
 *   vbs       [Nc] int32, each in [0, 64]
 *   topk      ids per row written to topk_idx, in [1, Nc]; ignored when
 *             topk_idx is NULL
 *   topk_idx  [B][NH][Nc][topk] int32 device output or NULL; when given it is
 *             exactly what vsa_select writes for the same inputs
 *   sm_scale  softmax scale of the coarse scores; <= 0 selects 1/sqrt(D);
 *             must be finite
 *   o_coarse  [B][NH][Nc][D] float32 device output
 *   workspace >= vsa_coarse_workspace_bytes(B, NH, Nc, D) bytes, 256-byte
 *             aligned, not overlapping the tensors; on return it holds Qc, Kc,
 *             S and Vc (layout not part of the interface)
 * q_tiled, k_tiled, v_tiled and o_coarse must be 16-byte aligned. Errors:
 * VSA_ERR_NULL, VSA_ERR_SHAPE, VSA_ERR_UNSUPPORTED (D, alignment, Nc >
 * VSA_MAX_CUBES), VSA_ERR_RANGE (topk, sm_scale), VSA_ERR_WORKSPACE,
 * VSA_ERR_HIP. */
int32_t vsa_coarse(const vsa_bf16_t* q_tiled, const vsa_bf16_t* k_tiled,
                   const vsa_bf16_t* v_tiled, const int32_t* vbs, int32_t B, int32_t Nc,
                   int32_t NH, int32_t D, int32_t topk, int32_t* topk_idx, float sm_scale,
                   float* o_coarse, void* workspace, size_t workspace_bytes,
                   vsa_stream_t stream);

/* Gated combine of the two stages. VSA blog, "Two-Stage Architecture" (the
 * final output mixes the coarse-stage and fine-stage outputs through
 * learnable gates). For every token row s of cube c = s / 64, head h and
 * channel d:
 *   out[b][s][h][d] = bf16(gate_coarse[b][s][h][d] * o_coarse[b][h][c][d]
 *                          + gate_fine[b][s][h][d] * o_fine[b][s][h][d])
 * evaluated in fp32 (one fused multiply-add over the fine product) and
 * rounded to nearest even.
 *   o_fine, gate_coarse, gate_fine, out  [B][Nc*64][NH][D] bf16, tiled order;
 *             out may be the same buffer as o_fine or as a gate (each element
 *             is read before it is written), otherwise no overlap
 *   o_coarse  [B][NH][Nc][D] float32 (vsa_coarse's output)
 * All pointers must be 16-byte aligned. Errors: VSA_ERR_NULL, VSA_ERR_SHAPE,
 * VSA_ERR_UNSUPPORTED, VSA_ERR_HIP. */
int32_t vsa_gate_combine(const vsa_bf16_t* o_fine, const float* o_coarse,
                         const vsa_bf16_t* gate_coarse, const vsa_bf16_t* gate_fine,
                         vsa_bf16_t* out, int32_t B, int32_t Nc, int32_t NH, int32_t D,
                         vsa_stream_t stream);

/* Block mask -> lookup table (VSA blog, "Sparse Encoding in CK Tile": Jenga
 * keeps the full block relation matrix B and skips cells with B[i][j] = 0;
 * VSA keeps the selected block ids and a valid count per query block). For
 * every row r = (b, h, i) of block_mask:
 *   kv_block_idx[r][0 .. n)  = the ids j with block_mask[r][j] != 0, ascending
 *   valid_block_num[r]       = n = min(number of such j, max_kv)
 * Entries of kv_block_idx[r] at positions >= n are not written. A row with
 * more than max_kv set cells keeps its max_kv lowest ids and adds 1 to
 * *n_truncated (a device int32 the caller zeroes first; may be NULL).
 *   block_mask       [B][NH][Nq][Nkv] uint8 device array (any nonzero = set)
 *   kv_block_idx     [B][NH][Nq][max_kv] int32 device output
 *   valid_block_num  [B][NH][Nq] int32 device output
 * The output feeds vsa_fwd_lut directly. Errors: VSA_ERR_NULL, VSA_ERR_SHAPE,
 * VSA_ERR_RANGE (max_kv outside [1, Nkv]), VSA_ERR_HIP. */
int32_t vsa_mask_to_lut(const uint8_t* block_mask, int32_t B, int32_t NH, int32_t Nq,
                        int32_t Nkv, int32_t max_kv, int32_t* kv_block_idx,
                        int32_t* valid_block_num, int32_t* n_truncated, vsa_stream_t stream);

/* Checks the vsa_fwd precondition on topk_idx on the device: counts, into
 * *bad_count (one int32 in device memory, which the caller zeroes first), the
 * entries that are outside [0, Nkv) or repeat an earlier id of their row
 * (VSA blog, "Block-Sparse Encoding": the index list names each selected
 * key/value block once). Errors: VSA_ERR_NULL, VSA_ERR_SHAPE,
 * VSA_ERR_UNSUPPORTED, VSA_ERR_RANGE, VSA_ERR_HIP. */
int32_t vsa_validate_topk(const int32_t* topk_idx, int32_t B, int32_t NH,
                          int32_t Nq, int32_t Nkv, int32_t topk,
                          int32_t* bad_count, vsa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H */
