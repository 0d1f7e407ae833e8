/*
 * tdx.h - C ABI of the collective KV-cache reuse kernels for AMD MI355X (gfx950).
 *
 * The operations follow the TokenDance pages' statement of the problem.  In
 * one synchronous multi-agent round every agent i's prompt is its private
 * history followed by the same shared output blocks in an agent-specific
 * order (TokenDance deep-dive notes, Summary "Motivation", Figure 1), so one
 * shared block sits at a different absolute offset in every prompt.  The
 * library provides:
 *
 *   tdx_rerotate          one batched RoPE correction of the cached shared K
 *                         to all N agents' offsets (notes, Summary "Method",
 *                         Figure 7 path T3, Deep Analysis §0).
 *   tdx_select_important  one check-layer key-difference pass over the group,
 *                         one important-position set and the least-deviation
 *                         Master (notes, Summary "Method", §3c A2/A3).
 *   tdx_diff_encode       Master-Mirror block-sparse diff: per Mirror and
 *                         layer, the indices and K/V values of the 16-token
 *                         blocks that differ from the Master (notes, Figure 8,
 *                         §2b; blog §4.3).
 *   tdx_restore_attn      fused restore: diff blocks merged into Master tiles
 *                         and RoPE recovered inside the decode-attention
 *                         kernel, no dense Mirror written (notes §3d, §4
 *                         "Fused Diff Restore"; blog §4.4).
 *   tdx_restore_dense +   the dense comparator: materialise every agent's
 *   tdx_decode_attn_dense cache, then attend (notes §3d, §7b).
 *   tdx_restore_transfer  the transfer-path restore: Mirrors rebuilt layer by
 *                         layer from a Master and diff records kept in host
 *                         storage (notes §3d Algorithm 1; blog §4.4).
 *   tdx_*_paged           the four collective calls over a paged KV pool
 *                         (16-token pages + page tables; notes §3c, §3d).
 *   tdx_round_plan_*      host side: shared blocks, groups and their layouts
 *                         derived from the requests' token IDs (notes §4
 *                         Round-Aware Prompt Interface, §5 "Scheduling").
 *
 * Conventions shared by every call
 *  - Tensor arguments are DEVICE pointers (tdx_restore_transfer also takes
 *    pinned host storage) to dense row-major arrays owned by the caller; the
 *    library allocates and frees nothing and keeps no state apart from a
 *    thread-local error string and the static scratch array of
 *    tdx_select_important_noalloc.  Scratch memory is passed as
 *    (ws, ws_bytes), sized by the matching tdx_*_workspace() query.
 *  - Element type of K, V, q and outputs is shape->dtype (fp32 or bf16 bit
 *    patterns).  All tensor pointers must be 16-byte aligned.
 *  - RoPE is the rotate-half form: dims (e, e + D/2) form a pair rotated by
 *    angle p * theta^(-2e/D).  Cos/sin of each shift are evaluated in double
 *    precision and applied in fp32.
 *  - stream is a hipStream_t passed as void* (NULL = default stream).  Every
 *    call only enqueues work; results are valid after the stream completes.
 *  - All argument checks run before anything is enqueued: a call that
 *    returns an error has had no effect.  Launch failures return TDX_EHIP.
 *    tdx_last_error() gives the calling thread's last error message.
 */
#ifndef TDX_H
#define TDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TDX_VERSION 10000 /* 1.0.0 */
#define TDX_DIFF_BLOCK 16 /* tokens per diff block (notes §3c A4: 16/32-token pages) */

enum {
  TDX_OK = 0,
  TDX_EINVAL = -1,       /* bad argument: null/unaligned pointer, bad size or shape */
  TDX_EUNSUPPORTED = -2, /* shape outside what the kernels are built for */
  TDX_EHIP = -3,         /* a HIP runtime call or kernel launch failed */
  TDX_EINTERNAL = -4,    /* unexpected internal failure */
  TDX_EWORKSPACE = -5    /* ws is null or ws_bytes below the workspace query */
};

typedef enum { TDX_F32 = 0, TDX_BF16 = 1 } tdx_dtype;

/* Model-side shape.  n_layers is the layer count of the K/V arrays passed to
 * the call; head_dim is 64 or 128; n_q_heads is a multiple of n_kv_heads
 * (query head hq reads KV head hq / (n_q_heads / n_kv_heads)). */
typedef struct {
  int32_t n_layers;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t head_dim;
  int32_t dtype;     /* tdx_dtype */
  double rope_theta; /* RoPE base theta > 1 */
} tdx_shape;

/* Round geometry.  Shared tokens are kept in canonical order: block b covers
 * canonical tokens [blk_start[b], blk_start[b+1]).  src_pos[b] is the absolute
 * position the cached K of block b was rotated at; dst_pos[i*B + b] is the
 * absolute position of block b's first token in agent i's prompt.  Agent i
 * needs its block b shifted by Delta(i,b) = dst_pos[i*B+b] - src_pos[b].
 * The three arrays are DEVICE int32 arrays; n_tokens == blk_start[B]. */
typedef struct {
  int32_t n_agents; /* N >= 1 */
  int32_t n_blocks; /* B >= 1 */
  int32_t n_tokens; /* T >= 1 */
  const int32_t *blk_start; /* [B+1], non-decreasing, blk_start[0] = 0 */
  const int32_t *src_pos;   /* [B] */
  const int32_t *dst_pos;   /* [N*B] */
} tdx_layout;

/* ---- a1: batched RoPE delta re-rotation ---------------------------------
 * k_out[i][l][t][h][:] = round(R(Delta(i, b(t))) . k_cached[l][t][h][:]) for
 * every agent i, layer l < n_layers, canonical token t, KV head h: one
 * launch for the whole group (notes, Summary "Method"; Figure 7 T3).  V is
 * never rotated.  A block with Delta = 0 is copied bit for bit.
 *   k_cached  [L][T][Hkv][D]      read once
 *   k_out     [N][L][T][Hkv][D]   written, tokens in canonical order
 * Block lengths may be any non-negative integers.  Returns TDX_OK or an
 * error; no workspace. */
int tdx_rerotate(const tdx_shape *shape, const tdx_layout *layout,
                 const void *k_cached, void *k_out, void *stream);

/* ---- a2 + a3: check-layer key difference, one important set, Master -----
 * At the check layer (notes, Summary "Method"; CacheBlend-style deviation):
 *   dev[i][t]    = sum_h || k_recomp[i][t][h] - k_reuse[i][check][t][h] ||_2
 *   score[t]     = sum_i dev[i][t]            (fp32, from double sums)
 *   agent_dev[i] = sum_t dev[i][t]            (fp32, from double sums)
 *   selected[0..k) = the k largest score[t], ties to the lower t, ascending
 *   master[0]    = argmin_i agent_dev[i] (fp32 values), ties to the lower i
 * The one set is reused by every later layer and never recomputed (notes
 * §3c A3); the least-deviation agent keeps the full cache (§3c A2).
 *   k_reuse   [N][L][T][Hkv][D]  re-rotated K (e.g. tdx_rerotate output);
 *             the slice at layer check_layer is read
 *   k_recomp  [N][T][Hkv][D]     recomputed K at the check layer
 *   k         1 <= k <= T (tdx_topk_count gives ceil(pct * T / 100))
 *   dev [N][T], score [T], agent_dev [N] (fp32); selected [k], master [1]
 *   (int32) - all device, all written.
 * Deterministic: every reduction runs in a fixed order. */
int tdx_select_important(const tdx_shape *shape, const tdx_layout *layout,
                         int32_t check_layer, const void *k_reuse,
                         const void *k_recomp, int32_t k, float *dev,
                         float *score, float *agent_dev, int32_t *selected,
                         int32_t *master, void *ws, size_t ws_bytes,
                         void *stream);
size_t tdx_select_workspace(const tdx_shape *shape, const tdx_layout *layout);

/* tdx_select_important for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops and harnesses that forbid hipMalloc.
 * Same arguments, outputs and checks as tdx_select_important minus the
 * workspace: the scratch (tdx_select_workspace bytes) is a static device
 * array of TDX_SELECT_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends.  The call allocates nothing; it uses the array of
 * the calling thread's current device (stream must belong to that device).
 *  - A round whose workspace exceeds TDX_SELECT_SCRATCH_BYTES is rejected
 *    with TDX_EUNSUPPORTED before anything is enqueued.
 *  - The first call on a device looks the array's address up once (a HIP
 *    runtime query, no allocation); a failure returns TDX_EHIP.
 *  - Every call on one GPU shares that GPU's array: calls that overlap on
 *    one GPU (two streams, two threads) race and must be serialised by the
 *    caller.  Nothing in the array needs to start at zero; each call
 *    overwrites what it reads. */
#define TDX_SELECT_SCRATCH_BYTES (4u << 20) /* 4 MiB: N * ceil(T / 4) * 8 bytes */
int tdx_select_important_noalloc(const tdx_shape *shape, const tdx_layout *layout,
                                 int32_t check_layer, const void *k_reuse,
                                 const void *k_recomp, int32_t k, float *dev,
                                 float *score, float *agent_dev,
                                 int32_t *selected, int32_t *master,
                                 void *stream);
/* ceil(pct * n_tokens / 100) in integer arithmetic, clamped to [1, n_tokens];
 * returns 0 when n_tokens < 1 or pct is outside [0, 100]. */
int32_t tdx_topk_count(int32_t pct, int32_t n_tokens);

/* ---- a4: Master-Mirror block-sparse diff encode ---------------------------
 * For every agent i != *master and layer l, the 16-token blocks beta of its
 * canonical-frame cache whose K or V differs from the Master's in any stored
 * bit (all heads, all dims) are recorded as one CSR row r = i*L + l (notes,
 * Figure 8: Diff = block-sparse (indices, values); §2b one record per Mirror
 * per layer).  The values are the Mirror's own K/V (a replacement, so
 * decoding is lossless).  The Master's rows are empty.
 *   master      [1] device int32 (e.g. tdx_select_important output)
 *   agents_k/v  [N][L][T][Hkv][D] canonical-frame caches; T % 16 == 0
 *   cap_blocks  capacity of diff_idx / diff_k / diff_v in blocks (>= 0)
 *   diff_off    [N*L+1] int32, row offsets, always written in full and
 *               clamped to cap_blocks (diff_off[r] = min(true offset, cap))
 *   diff_idx    [cap] int32, ascending block indices within each row
 *   diff_k/v    [cap][16][Hkv][D]
 *   nnz         [1] int64: the true total; when it exceeds cap_blocks the
 *               entries at positions >= cap_blocks are not written, which the
 *               caller detects by reading nnz (a device-side condition).  The
 *               clamped offsets name written entries only, so an overflowed
 *               record is still safe to pass to the restore calls (no read
 *               past the capacity); it is incomplete: the dropped blocks of
 *               a Mirror restore as the Master's.
 *               nnz = -1 (and every row empty) when *master is not in [0, N).
 *   master_k_out/master_v_out  [L][T][Hkv][D] dense copy of the Master, or
 *               NULL to skip. */
int tdx_diff_encode(const tdx_shape *shape, const tdx_layout *layout,
                    const int32_t *master, const void *agents_k,
                    const void *agents_v, int64_t cap_blocks, int32_t *diff_off,
                    int32_t *diff_idx, void *diff_k, void *diff_v,
                    int64_t *nnz, void *master_k_out, void *master_v_out,
                    void *ws, size_t ws_bytes, void *stream);
size_t tdx_diff_encode_workspace(const tdx_shape *shape, const tdx_layout *layout);

/* ---- a5: fused restore + decode attention --------------------------------
 * out[i][l][hq] = sum_j softmax_j(scale * q[i][l][hq] . key_j) val_j over
 * agent i's private keys followed by its shared keys, where the shared key of
 * canonical token t is R(Delta(i, b(t))) applied to K~_i[l][t], and K~_i / V~_i
 * are the Master patched with agent i's diff rows.  The patch and the RoPE
 * recovery happen tile by tile inside the attention kernel; no dense Mirror
 * is written (notes §3d, §4; blog §4.4).
 *   q          [N][L][Hq][D]
 *   priv_off   [N+1] device int32 offsets into the private arrays
 *   priv_k/v   [L][P_total][Hkv][D], agent i owns rows priv_off[i]..priv_off[i+1]
 *   max_priv   host scalar >= max_i (priv_off[i+1] - priv_off[i]); a longer
 *              history is attended only up to its first max_priv tokens
 *   master_k/v the Master's cache, [L][T][Hkv][D] (T % 16 == 0), found at
 *              master_k + m * master_stride elements (same for v), where
 *              m = *master_sel (device int32, clamped to [0, N)) or m = 0 when
 *              master_sel is NULL.  Pass the dense copy written by
 *              tdx_diff_encode with master_sel = NULL, or read the Master in
 *              place: master_k = agents_k, master_sel = the Master chosen by
 *              tdx_select_important, master_stride = L*T*Hkv*D (the Master
 *              keeps its own cache, notes Figure 8).
 *   diff_off / diff_idx / diff_k / diff_v  as written by tdx_diff_encode
 *   scale      softmax scale (> 0), usually 1/sqrt(D)
 *   out        [N][L][Hq][D]
 * Returns TDX_EUNSUPPORTED when N * L * (ceil(max_priv / 16) + T / 16), the
 * number of 16-token tiles the call plans, exceeds 2^31 - 1 (the same bound
 * holds for tdx_restore_attn_paged and tdx_decode_attn_dense, whose
 * workspace queries then return 0). */
int tdx_restore_attn(const tdx_shape *shape, const tdx_layout *layout,
                     const void *q, const int32_t *priv_off,
                     const void *priv_k, const void *priv_v, int32_t max_priv,
                     const void *master_k, const void *master_v,
                     const int32_t *master_sel, int64_t master_stride,
                     const int32_t *diff_off, const int32_t *diff_idx,
                     const void *diff_k, const void *diff_v, float scale,
                     void *out, void *ws, size_t ws_bytes, void *stream);
size_t tdx_restore_attn_workspace(const tdx_shape *shape, const tdx_layout *layout,
                                  int32_t max_priv);

/* ---- transfer-path restore (Mirrors rebuilt from host storage) -------------
 * The pages' restore path (notes Summary "Method" and §3d Algorithm 1 "Fused
 * Diff Restore"; blog §4.4): the Master and the Mirrors' diff records live in
 * storage outside the GPU and an agent's KV is rebuilt layer by layer on the
 * way in, merged block by block and RoPE-recovered, with no dense Mirror in
 * between.  For every requested agent a = agents[j] and layer l in
 * [layer_begin, layer_end):
 *   k_out[j][l][t] = round(R(Delta(a, b(t))) K~_a[l][t]),  v_out[j][l][t] = V~_a[l][t]
 * with K~_a / V~_a the Master patched with agent a's diff rows (the same rows
 * tdx_restore_dense writes for agent a; a zero shift copies the bits).  Layers outside the range are not
 * written.  The kernels read the Master and the diff record directly where
 * they are, so they may sit in pinned host memory (hipHostMalloc, or a
 * pinned torch tensor: the reads then cross PCIe, once per block for all
 * requested agents) or in device memory; pageable host memory is rejected
 * with TDX_EINVAL.
 *   master_k/v       [L][T][Hkv][D] (T % 16 == 0), host-pinned or device
 *   diff_off / diff_idx / diff_k / diff_v  as written by tdx_diff_encode,
 *                    host-pinned or device
 *   agents           device int32 [n_req], each in [0, N) (values outside are
 *                    clamped to it); n_req >= 1
 *   k_out/v_out      device [n_req][L][T][Hkv][D]
 *   ws               tdx_restore_transfer_workspace(shape, layout, n_req,
 *                    layer_begin, layer_end) bytes (device) */
int tdx_restore_transfer(const tdx_shape *shape, const tdx_layout *layout,
                         const void *master_k, const void *master_v,
                         const int32_t *diff_off, const int32_t *diff_idx,
                         const void *diff_k, const void *diff_v,
                         const int32_t *agents, int32_t n_req,
                         int32_t layer_begin, int32_t layer_end,
                         void *k_out, void *v_out, void *ws, size_t ws_bytes,
                         void *stream);
size_t tdx_restore_transfer_workspace(const tdx_shape *shape, const tdx_layout *layout,
                                      int32_t n_req, int32_t layer_begin, int32_t layer_end);

/* ---- a6: dense comparator --------------------------------------------------
 * tdx_restore_dense writes every agent's full cache:
 *   k_dense[i][l][t] = round(R(Delta(i, b(t))) K~_i[l][t]), v_dense[i][l][t] = V~_i[l][t]
 * ([N][L][T][Hkv][D] each; inputs as for tdx_restore_attn).  R(0) is the
 * identity: the K rows of a block with Delta = 0 are copied bit for bit (as
 * in tdx_rerotate and tdx_restore_transfer).
 * tdx_decode_attn_dense then runs plain decode attention of agent i over its
 * private keys followed by k_dense[i] / v_dense[i] (outputs as tdx_restore_attn).
 * Together they are the dense restore-then-attend path the fused restore is
 * measured against (notes §3d, §7b). */
int tdx_restore_dense(const tdx_shape *shape, const tdx_layout *layout,
                      const void *master_k, const void *master_v,
                      const int32_t *master_sel, int64_t master_stride,
                      const int32_t *diff_off, const int32_t *diff_idx,
                      const void *diff_k, const void *diff_v, void *k_dense,
                      void *v_dense, void *stream);
int tdx_decode_attn_dense(const tdx_shape *shape, const tdx_layout *layout,
                          const void *q, const int32_t *priv_off,
                          const void *priv_k, const void *priv_v,
                          int32_t max_priv, const void *k_dense,
                          const void *v_dense, float scale, void *out,
                          void *ws, size_t ws_bytes, void *stream);
size_t tdx_decode_attn_dense_workspace(const tdx_shape *shape, const tdx_layout *layout,
                                       int32_t max_priv);

/* ---- paged KV layout ---------------------------------------------------------
 * The four collective calls over caches kept in a serving KV pool: 16-token
 * pages plus page tables instead of contiguous canonical arrays (notes §3c A4
 * and §3d: 16/32-token pages, diff indices aligned to page boundaries, the
 * fused restore's dependence on the paged KV slot map; §5 "Scheduling":
 * memory management inherits paged attention).  Every sequence keeps its
 * tokens in the order the contiguous calls use (a canonical shared region is
 * ceil(T/16) pages, page j holding canonical tokens 16j .. 16j+15), so a
 * 16-token diff block is exactly one page.
 *
 * A pool holds n_layers x n_pages pages: page p of layer l is the 16 x Hkv x D
 * elements at pool + (l * n_pages + p) * 16 * Hkv * D (shape->dtype), the same
 * page ID in every layer.  Row r of a page table lists one sequence's pages
 * at pages + r * stride.  Page IDs are read on the device; IDs outside
 * [0, n_pages) are clamped, so a bad table can read or write a wrong page of
 * the pool but never memory outside it.  Output pages of different sequences
 * must be distinct; input and output pools may be the same allocation. */
typedef struct {
  void *k_pool;          /* K pool, 16-byte aligned */
  void *v_pool;          /* V pool, same layout; NULL where the call reads only K */
  int64_t n_pages;       /* pages per layer in each pool, >= 1 */
  const int32_t *pages;  /* device page table, 4-byte aligned */
  int64_t stride;        /* entries between consecutive rows (>= a row's pages when rows > 1) */
} tdx_paged_kv;

/* a1 paged: out row i's pages receive agent i's re-rotated K, as
 * tdx_rerotate writes k_out[i]; cached row 0 lists the cached K's pages.  A
 * partial last page (T % 16 != 0) is written only up to T. */
int tdx_rerotate_paged(const tdx_shape *shape, const tdx_layout *layout, const tdx_paged_kv *cached,
                       const tdx_paged_kv *out, void *stream);
/* a2 + a3 paged: agent i's re-rotated K at check_layer is row i of k_reuse;
 * everything else as tdx_select_important (same workspace size). */
int tdx_select_important_paged(const tdx_shape *shape, const tdx_layout *layout, int32_t check_layer,
                               const tdx_paged_kv *k_reuse, const void *k_recomp, int32_t k, float *dev,
                               float *score, float *agent_dev, int32_t *selected, int32_t *master, void *ws,
                               size_t ws_bytes, void *stream);
/* a4 paged: agent i's canonical K/V (T/16 pages, K and V pools under one
 * table) is row i of agents.  The record is diff_off and diff_idx as in
 * tdx_diff_encode plus diff_page[e], the Mirror's own page holding entry e's
 * block: the values stay in the pool (the Mirror's other pages can be
 * released).  When diff_k/diff_v are set, the values are also copied there as
 * in tdx_diff_encode.  Same workspace size as tdx_diff_encode. */
int tdx_diff_encode_paged(const tdx_shape *shape, const tdx_layout *layout, const int32_t *master,
                          const tdx_paged_kv *agents, int64_t cap_blocks, int32_t *diff_off, int32_t *diff_idx,
                          int32_t *diff_page, void *diff_k, void *diff_v, int64_t *nnz, void *ws, size_t ws_bytes,
                          void *stream);
/* a5 paged: as tdx_restore_attn with agent i's private history in row i of
 * priv (ceil(max_priv/16) entries per row, lengths from priv_off, history
 * past max_priv never read; unused when max_priv = 0),
 * the Master as row *master_sel of agents (row 0 when master_sel is NULL; the
 * selector is clamped to [0, N)) and diff entry e's values in page
 * diff_page[e] of the agents' pools.  Same workspace size as
 * tdx_restore_attn. */
int tdx_restore_attn_paged(const tdx_shape *shape, const tdx_layout *layout, const void *q,
                           const int32_t *priv_off, const tdx_paged_kv *priv, int32_t max_priv,
                           const tdx_paged_kv *agents, const int32_t *master_sel, const int32_t *diff_off,
                           const int32_t *diff_idx, const int32_t *diff_page, float scale, void *out, void *ws,
                           size_t ws_bytes, void *stream);

/* NEXT-1 over pages: as tdx_restore_transfer, with requested agent j's
 * rebuilt K (re-rotated) and V written into the pages of row j of out (T/16
 * entries per row, canonical order, both pools) instead of a dense array:
 * the Master chunk and the diff blocks go straight into the paged KV of the
 * agent (notes §2a stage table, "Fused restore"; §3d).  Pages not listed in
 * the rows, and layers outside [layer_begin, layer_end), are not written. */
int tdx_restore_transfer_paged(const tdx_shape *shape, const tdx_layout *layout, const void *master_k,
                               const void *master_v, const int32_t *diff_off, const int32_t *diff_idx,
                               const void *diff_k, const void *diff_v, const int32_t *agents, int32_t n_req,
                               int32_t layer_begin, int32_t layer_end, const tdx_paged_kv *out, void *ws,
                               size_t ws_bytes, void *stream);

/* ---- round structure from token IDs (host only) -----------------------------
 * The step before the collective calls: find the blocks that the requests of
 * one round share and derive, per group of compatible requests, the
 * tdx_layout arrays.  TokenDance notes §4 "Key Innovations" (Round-Aware
 * Prompt Interface: a reserved separator token marks logical block
 * boundaries and the runtime hashes segment content, not positions), §2a
 * (data flow: prompt assembly with separators, segment hashing, grouping of
 * compatible requests), §5 "Scheduling" (a group needs the same cached span
 * and disjoint slot mappings; other requests fall back to per-request reuse);
 * blog §4.1 (the separator).
 *
 * Definitions:
 *  - a segment is a maximal run of tokens != sep_token in one request;
 *    separators belong to no segment (they are private tokens);
 *  - segments with equal token sequences are one block (exact comparison;
 *    the hash only indexes candidates).  Block IDs are dense, numbered in
 *    order of first appearance (requests in order, segments in order);
 *  - a block is shared when at least min_share distinct requests hold it
 *    (min_share <= 0: every request).  In one request only the first
 *    occurrence is the shared copy; repeats are private;
 *  - requests holding the same set of shared blocks form one group, unless
 *    slot ranges are given: a request then joins the first group of its set
 *    (groups numbered by first member) none of whose members' half-open
 *    ranges [slot_begin, slot_end) intersects its own, else a new group;
 *  - a group's blocks are ordered as they first appear in its first member:
 *    blk_start is the prefix sum of their lengths, src_pos[b] = blk_start[b]
 *    (the cached K of a block sits at its canonical position), dst_pos[i][b]
 *    is the offset of block b's shared copy in member i, priv_len[i] = the
 *    member's length - T.  A group of one request is the per-request case.
 *
 * All pointers are HOST pointers.  tokens [req_off[n_req]] int32 (request r
 * is tokens[req_off[r] .. req_off[r+1])), req_off [n_req+1] non-decreasing
 * int64; slot_begin/slot_end [n_req] int64 or both NULL.  On success *plan
 * owns the result until tdx_round_plan_free.  Errors: TDX_EINVAL (null or
 * inconsistent arguments, a request or shared region over INT32_MAX tokens;
 * *plan is then NULL), TDX_EINTERNAL (out of host memory).  The encode and
 * restore calls further need T % 16 == 0, which a derived layout need not
 * meet. */
typedef struct tdx_round_plan tdx_round_plan;
int tdx_round_plan_build(const int32_t *tokens, const int64_t *req_off, int32_t n_req, int32_t sep_token,
                         int32_t min_share, const int64_t *slot_begin, const int64_t *slot_end,
                         tdx_round_plan **plan);
/* number of groups (>= 1), or TDX_EINVAL for a NULL plan */
int tdx_round_plan_n_groups(const tdx_round_plan *plan);
/* N, B and T of group g; any output may be NULL */
int tdx_round_plan_group_dims(const tdx_round_plan *plan, int32_t group, int32_t *n_agents,
                              int32_t *n_blocks, int32_t *n_tokens);
/* group g's members (request indices, ascending) [N], block IDs [B],
 * blk_start [B+1], src_pos [B], dst_pos [N*B] (member-major), priv_len [N];
 * any output may be NULL */
int tdx_round_plan_group(const tdx_round_plan *plan, int32_t group, int32_t *agents, int32_t *seg_ids,
                         int32_t *blk_start, int32_t *src_pos, int32_t *dst_pos, int32_t *priv_len);
/* request r's group, and its token map [req_off[r+1] - req_off[r]]: the
 * canonical index of each token in its group's shared region, -1 for a
 * private token; either output may be NULL */
int tdx_round_plan_request(const tdx_round_plan *plan, int32_t request, int32_t *group, int32_t *token_map);
void tdx_round_plan_free(tdx_round_plan *plan);

/* ---- utilities -------------------------------------------------------------*/
const char *tdx_strerror(int code); /* static text for a return code */
const char *tdx_last_error(void);   /* detail of the calling thread's last error */
int tdx_version(void);              /* TDX_VERSION */

#ifdef __cplusplus
}
#endif
#endif /* TDX_H */
