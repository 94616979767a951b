/*
 * libsla — forward pass of sparse-linear hybrid attention on AMD MI355X (gfx950).
 *
 * The method (SLA analysis page for arXiv 2509.24006; "2025稀疏注意力架构综述",
 * section 10 SLA and section 11 SpargeAttn prediction formulas):
 *   1. predict:  mean-pool Q and K over 64-token blocks and score every
 *                (query block, key block) pair with the pooled vectors;
 *   2. classify: per query-block row the top share of key blocks is critical,
 *                the bottom share negligible, the rest marginal;
 *   3. execute:  critical pairs get exact softmax attention, marginal pairs
 *                linear attention with phi = elu + 1 through per-key-block
 *                states H_j = phi(K_j)^T V_j and z_j = sum phi(K_j),
 *                negligible pairs are skipped;
 *   4. combine:  O = O_sparse + Proj(O_linear), Proj a learned linear layer on
 *                the linear branch (the identity unless a weight is passed).
 * Smooth-K (the open-source code's zero-mean K, SLA analysis page) is available
 * for the linear branch: sla_key_mean, then sla_linear_kv_reduce with k_shift.
 * Variants: the SALAD gated linear branch over all keys (SALAD page, method
 * framework) and an NSA-style selected-block + sliding-window causal branch
 * whose block selection is shared by a GQA group ("Sparse Attention 方法综述",
 * section 2 NSA and its key-parameter table).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named in an sla_tensor, and every float / int buffer argument, are
 *   DEVICE pointers owned by the caller.  The library keeps no pointer after a
 *   call returns and allocates no device memory: scratch space comes in through
 *   `workspace` arguments sized by the matching *_workspace_bytes() query.
 * - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *   NULL = the null stream).  The caller keeps every buffer alive until the
 *   stream has passed the work.  Calls never synchronise.
 * - Arguments are validated on the host before anything is launched; an invalid
 *   argument returns an error code and launches nothing.  A failed launch
 *   returns SLA_ERR_HIP.  Device faults surface at the caller's next sync.
 * - Q, K, V use layout [B, H, N, d] with element strides (sB, sH, sN) and unit
 *   d-stride; rows are 16-byte aligned and sN <= SLA_MAX_ROW_STRIDE (larger row
 *   strides return SLA_ERR_UNSUPPORTED).  d is 64 or 128, the block size is 64,
 *   N is a multiple of 64 and at most one block is partial:
 *   N - 64 < n_valid <= N.  Positions >= n_valid are padding: they are excluded
 *   from pooled means and from both attention branches, and the output rows of
 *   padded queries are written as zeros.
 * - All library outputs are dense row-major arrays with the shapes stated.
 * - The calls are reentrant and keep no global mutable state.
 */
#ifndef SLA_H
#define SLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SLA_ABI_VERSION 6
#define SLA_BLOCK 64
#define SLA_MAX_KEY_BLOCKS 4096 /* per row: N <= 262144 tokens */
#define SLA_MAX_ROW_STRIDE (1 << 24) /* elements between consecutive tokens of one head */

typedef int32_t sla_status;
enum {
  SLA_OK = 0,
  SLA_ERR_NULL = 1,        /* a required pointer is NULL */
  SLA_ERR_SHAPE = 2,       /* inconsistent or unsupported sizes */
  SLA_ERR_ALIGN = 3,       /* a pointer or row stride is not 16-byte aligned */
  SLA_ERR_RANGE = 4,       /* a count, share or length is out of range */
  SLA_ERR_UNSUPPORTED = 5, /* valid but unsupported combination */
  SLA_ERR_CAPACITY = 6,    /* an output capacity is too small */
  SLA_ERR_HIP = 7,         /* a HIP launch failed */
  SLA_ERR_WORKSPACE = 8    /* workspace missing or smaller than required */
};

enum { SLA_BF16 = 0, SLA_F32 = 1 };

/* Linear-branch modes of sla_attn_fwd. */
enum {
  SLA_LIN_NONE = 0,         /* sparse branch only (NSA-style selected + window) */
  SLA_LIN_MARGINAL = 1,     /* SLA: linear attention over each row's marginal blocks */
  SLA_LIN_GLOBAL_GATED = 2, /* SALAD: gated linear attention over all valid keys */
  SLA_LIN_ROW_STATES = 3    /* SLA with the per-row sums precomputed by sla_marginal_states */
};

typedef struct {
  const void* ptr;       /* device pointer to element [0, 0, 0, 0] */
  int32_t dtype;         /* SLA_BF16 or SLA_F32 */
  int32_t B, H, N, d;
  int64_t sB, sH, sN;    /* element strides; the d stride is 1 */
} sla_tensor;

/* ABI version of the loaded library (SLA_ABI_VERSION of its build). */
int32_t sla_abi_version(void);

/* Static, human-readable name of a status code. Never NULL. */
const char* sla_status_str(sla_status s);

/*
 * Critical and negligible block counts of a row of nb candidates, from shares in
 * basis points (the pages give percentages per row; a fixed-budget top-k keeps the
 * same number per row — subquadratic sparse attention probe, reading notes).
 * n_crit = ceil(kh_bp * nb / 10000) (0 iff kh_bp == 0);
 * n_negl = min(floor(kl_bp * nb / 10000), nb - n_crit).
 * Host-only; returns SLA_ERR_RANGE unless 1 <= nb and 0 <= kh_bp, kl_bp <= 10000.
 */
sla_status sla_counts(int32_t nb, int32_t kh_bp, int32_t kl_bp, int32_t* n_crit, int32_t* n_negl);

/*
 * Prediction step (SpargeAttn prediction formulas in "2025稀疏注意力架构综述",
 * section 11; mean-pooled compressed prediction on the SLA analysis page).
 *
 *   q_pool[b,h,i,:]  = mean of the valid rows of block i of Q[b,h]   (fp32, [B,Hq,nb,d])
 *   k_pool[b,g,j,:]  = the same for K[b,g]                            (fp32, [B,Hkv,nb,d])
 *   scores[b,s,i,j]  = fp32( scale * (qsum . k_pool[b,g,j]) )         (fp32, [B,Hs,nb,nb])
 *     group_sum == 0: Hs = Hq, s = h, g = h / (Hq/Hkv), qsum = q_pool[b,h,i];
 *     group_sum != 0: Hs = Hkv, s = g, qsum = sum of q_pool[b,h,i] over the group's heads.
 *     Means and the dot product are taken in fp64; each stored value is rounded once.
 *     causal != 0: entries j > i are -inf.
 *   probs (nullable) = row softmax of scores over the row's finite candidates (fp32,
 *     same shape as scores), for diagnostics; the classification ranks the scores.
 * q and k share dtype and d; n_valid as in the conventions; scale > 0 (normally 1/sqrt(d)).
 * q_pool and k_pool are 16-byte aligned (SLA_ERR_ALIGN otherwise).
 * pooled (bit flags, 0 .. 3, SLA_ERR_RANGE otherwise):
 *   SLA_POOLED_K: k_pool already holds the key block means (written by sla_linear_kv_reduce's
 *     k_pool output, which reads K once for both); K's data is not read (its descriptor still
 *     gives the shapes);
 *   SLA_POOLED_Q: q_pool already holds the query block means (an earlier pooling-only call);
 *     Q's data is not read.
 * scores (nullable): NULL = pooling only (probs must be NULL too, no workspace needed), which
 *   with a later call that passes both pooled flags splits the pass into its pooling and its
 *   scoring kernels.
 * workspace: sla_pool_scores_workspace_bytes(...) bytes (the fp64 group sums of the pooled
 * queries, non-zero only with group_sum and more than one query head per KV head).
 */
#define SLA_POOLED_K 1
#define SLA_POOLED_Q 2
sla_status sla_pool_scores(const sla_tensor* q, const sla_tensor* k, int32_t n_valid,
                           int32_t group_sum, int32_t causal, float scale, int32_t pooled,
                           float* q_pool, float* k_pool, float* scores, float* probs,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes sla_pool_scores needs (B, Hq, Hkv, N, d, group_sum); 0 = none. */
size_t sla_pool_scores_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t d,
                                       int32_t group_sum);

/*
 * Smooth-K shift (SLA analysis page: the open-source code zero-means K, which the paper
 * does not mention): the mean of the valid key rows of each (batch, KV head),
 *   k_mean[b,g,r] = sum_j c_j * k_pool[b,g,j,r] / n_valid      (fp32, [B, Hkv, d])
 * with c_j = min(64, n_valid - 64 j) the valid rows of key block j, from the block means
 * k_pool [B, Hkv, nkb, d] that sla_pool_scores writes; summed in fp64, rounded once.
 * nkb * 64 - 64 < n_valid <= nkb * 64; d is 64 or 128; both pointers 16-byte aligned.
 * workspace: none.
 */
sla_status sla_key_mean(const float* k_pool, int32_t B, int32_t Hkv, int32_t nkb, int32_t d,
                        int32_t n_valid, float* k_mean, void* stream);

/*
 * Number of block-map index entries to allocate for `rows` rows (rows = B * Hs * nqb).
 * which = 0: critical (selected) list, which = 1: marginal list.  Non-causal maps are
 * exact (rows * n_crit and rows * (nkb - n_crit - n_negl)); causal maps return an upper
 * bound.  Returns -1 for invalid arguments.
 */
int64_t sla_block_map_capacity(int32_t B, int32_t Hs, int32_t nqb, int32_t nkb, int32_t n_crit,
                               int32_t n_negl, int32_t causal, int32_t window_tokens, int32_t which);

/* Workspace bytes sla_block_map needs (0 for non-causal maps). */
size_t sla_block_map_workspace_bytes(int32_t B, int32_t Hs, int32_t nqb, int32_t nkb, int32_t n_crit,
                                     int32_t causal, int32_t window_tokens);

/*
 * Classification step (three classes per Q-K block pair: SLA analysis page,
 * comparison tables; NSA selection and window: "Sparse Attention 方法综述", section 2).
 *
 * Input scores [B, Hs, nqb, nkb] fp32 (as written by sla_pool_scores).  Rows are
 * r = (b * Hs + s) * nqb + i.  Each row is ranked by one total order: score
 * descending, then key-block index ascending; -0.0 equals +0.0 and NaN ranks last.
 *
 * Non-causal (nqb, nkb any; n_crit + n_negl <= nkb):
 *   critical = first n_crit of the order, negligible = last n_negl, marginal = the rest.
 *   crit_rowptr[r] = r * n_crit, marg_rowptr[r] = r * (nkb - n_crit - n_negl).
 *   crit_flags (nullable) entries are 1.  marg_rowptr/marg_idx may both be NULL to skip
 *   the marginal list.  marg_bits (nullable): the marginal set of each row as a bit mask,
 *   [rows][ceil(nkb / 32)] uint32, block j = bit j % 32 of word j / 32 (the input of
 *   sla_marginal_states).
 * Causal (nqb == nkb, NSA-style): candidates are j <= i; the first min(n_crit, i + 1)
 *   of the order are selected (flag bit 0) and united with the window blocks
 *   max(0, i - floor((window_tokens + 62) / 64)) .. i (flag bit 1; none when
 *   window_tokens == 0).  n_negl is ignored, the marginal list is empty and its
 *   pointers may be NULL; marg_bits must be NULL.  Needs the workspace.
 *
 * Outputs (int32 unless stated): crit_rowptr [rows + 1], crit_idx [crit_cap] ascending
 * block indices per row, crit_flags [crit_cap] uint8, marg_rowptr [rows + 1],
 * marg_idx [marg_cap], row_counts [rows][3] = (critical, marginal, negligible).
 * crit_cap / marg_cap must be at least sla_block_map_capacity(...): SLA_ERR_CAPACITY.
 */
sla_status sla_block_map(const float* scores, int32_t B, int32_t Hs, int32_t nqb, int32_t nkb,
                         int32_t n_crit, int32_t n_negl, int32_t causal, int32_t window_tokens,
                         int32_t* crit_rowptr, int32_t* crit_idx, uint8_t* crit_flags, int64_t crit_cap,
                         int32_t* marg_rowptr, int32_t* marg_idx, int64_t marg_cap, uint32_t* marg_bits,
                         int32_t* row_counts, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free sla_block_map, for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, outputs, ownership and status codes as sla_block_map, minus the
 * workspace: the causal path stages its padded per-row lists in a static device array of the
 * library (16 MiB on every device the call runs on, held until the process ends; its address is
 * looked up once per device on the first call there, with that device current).
 * Limit: causal maps whose workspace (sla_block_map_workspace_bytes) exceeds 16 MiB return
 * SLA_ERR_WORKSPACE before any launch.  Non-causal maps use no scratch.
 * Concurrency: every call on one device shares that array, so calls that overlap on one device
 * (other streams, other host threads) race; order them on one stream.  Nothing in the array
 * needs clearing between calls (each call writes what it reads).  SLA_ERR_HIP if the device
 * or the array's address cannot be obtained.
 */
sla_status sla_block_map_noalloc(const float* scores, int32_t B, int32_t Hs, int32_t nqb, int32_t nkb,
                                 int32_t n_crit, int32_t n_negl, int32_t causal, int32_t window_tokens,
                                 int32_t* crit_rowptr, int32_t* crit_idx, uint8_t* crit_flags, int64_t crit_cap,
                                 int32_t* marg_rowptr, int32_t* marg_idx, int64_t marg_cap, uint32_t* marg_bits,
                                 int32_t* row_counts, void* stream);

/* Workspace bytes sla_linear_kv_reduce needs (non-zero only when the sums over all keys are wanted). */
size_t sla_kv_reduce_workspace_bytes(int32_t B, int32_t Hkv, int32_t N, int32_t d, int32_t want_blocks,
                                     int32_t want_all);

/*
 * Linear-attention key states (SLA analysis page: marginal pairs get linear attention,
 * O(N d^2); phi = elu + 1).  Per KV head and key block j, over the valid rows s:
 *   H[b,g,j,c,r] = sum_s phi(K[s,r]) * V[s,c]   (bf16 bits, [B, Hkv, nb, d, d]; nullable)
 *     i.e. each d x d state is stored transposed, V-feature major: (phi(K_j)^T V_j)^T,
 *     summed in fp32 and rounded once to bf16.
 *   z[b,g,j,r]   = sum_s phi(K[s,r])            (fp32, [B, Hkv, nb, d];     nullable with H)
 *   H_all[b,g]   = sum over all valid s          (fp32, [B, Hkv, d, d], same [c][r] layout; nullable)
 *   z_all[b,g]   = sum over all valid s          (fp32, [B, Hkv, d];        nullable with H_all)
 * k_shift (nullable, fp32 [B, Hkv, d], 16-byte aligned; smooth-K, normally from
 * sla_key_mean): when given, every phi(K[s,r]) above is phi(K[s,r] - k_shift[b,g,r]).
 * phi(K) is rounded to bf16 for the matrix-core contraction (fp32 accumulation); z sums
 * the same rounded values.  At least one of H, H_all must be non-NULL; outputs are 16-byte
 * aligned.
 * k_pool (nullable, fp32 [B, Hkv, nb, d], 16-byte aligned): also the key block means of the
 * prediction step, k_pool[b,g,j,:] = mean of the valid rows of block j of K[b,g] (raw K, no
 * shift), summed in fp64 and rounded once, the values sla_pool_scores writes (bit-identical
 * for bf16 K, whose fp64 block sums are exact; for fp32 K whenever a block's values lie within
 * 2^23 of each other in magnitude), so that sla_pool_scores with k_pooled skips reading K.  H_all needs a workspace of sla_kv_reduce_workspace_bytes(..., 1) bytes (fp32
 * partial sums over runs of consecutive key blocks, 4 to 32 of them by the shapes, then summed
 * in a fixed order).
 */
sla_status sla_linear_kv_reduce(const sla_tensor* k, const sla_tensor* v, int32_t n_valid,
                                const float* k_shift, void* H, float* z, float* H_all, float* z_all,
                                float* k_pool, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Marginal aggregation of one block map (marginal sets given as the bit masks sla_block_map
 * writes, [rows][ceil(nkb / 32)]): for every map row r with KV head g,
 *   S[r] = sum over marginal blocks j of H[b,g,j]  (bf16 bits, [rows, d, d], the [c][r] layout of H)
 *   u[r] = sum over marginal blocks j of z[b,g,j]  (fp32, [rows, d])
 * rows = B * Hs * nqb with Hs = Hkv if group_map else Hq; the KV head of map head s is
 * s if group_map else s / (Hq / Hkv).
 * H is the bf16 output of sla_linear_kv_reduce, z its fp32 z.
 * Computed as a 0/1 mask matrix product on the matrix cores: the bit masks expand to 0/1
 * operands, z is rounded to bf16 operands, sums accumulate in fp32 (deterministic) and S
 * is rounded once to bf16, the operand precision of the attention epilogue that reads it.
 * workspace: none.  sla_attn_fwd performs this step itself in SLA_LIN_MARGINAL mode.
 */
sla_status sla_marginal_states(const void* H, const float* z, int32_t B, int32_t Hq, int32_t Hkv,
                               int32_t nqb, int32_t nkb, int32_t d, int32_t group_map,
                               const uint32_t* marg_bits, void* S, float* u, void* stream);

/* Workspace bytes sla_attn_fwd needs for (B, Hs map heads, nqb query blocks, d, lin mode). */
size_t sla_attn_workspace_bytes(int32_t B, int32_t Hs, int32_t nqb, int32_t d, int32_t lin_mode);

/*
 * Attention step: exact block-sparse softmax attention over each query block's
 * critical list (FlashAttention-style online softmax; SLA analysis page, the
 * FlashAttn + linear attention pairing) plus the linear branch, summed
 * (O = O_sparse + Proj(O_linear); SLA analysis page, the zero-initialised Proj).
 *
 * For query row t of head h in block i, map row r = (b * Hs + s) * nqb + i with
 * s = h / (Hq/Hkv) if group_map else h, KV head g = h / (Hq/Hkv):
 *   O_sparse[t] = softmax over allowed keys of (scale * q_t . k_s) applied to v_s, or 0
 *     when no key is allowed.  Allowed: s < n_valid in a listed block; causal != 0 adds
 *     s <= t and (flag bit 0 of the block, or t - s < window_tokens).
 *   lin_mode SLA_LIN_MARGINAL (needs marg_bits, H (bf16) and z from sla_linear_kv_reduce):
 *     O_linear[t] = phi(q_t)^T S_r / (phi(q_t) . u_r), S_r and u_r the sums of H_j and
 *     z_j over row r's marginal blocks (computed as by sla_marginal_states); 0 when the
 *     row has none.
 *   lin_mode SLA_LIN_ROW_STATES: as SLA_LIN_MARGINAL, but H and z already hold the per-row
 *     sums S (bf16 bits, [rows, d, d]) and u (fp32, [rows, d]) written by sla_marginal_states
 *     for this map; marg_bits is not read and no workspace is needed.
 *   lin_mode SLA_LIN_GLOBAL_GATED (needs H_all, z_all, w_gate [Hq][d] fp32):
 *     O_linear[t] = sigmoid(q_t . w_gate[h]) * phi(q_t)^T H_all / (phi(q_t) . z_all).
 *   Proj (MARGINAL and ROW_STATES only; proj_w NULL = identity, then proj_b must be NULL):
 *     Proj(x) = W_h x + b_h on each valid row, W_h = proj_w[h'] a fp32 [d (out)][d (in)]
 *     row-major matrix and b_h = proj_b[h'] (nullable) fp32 [d], h' = 0 when
 *     proj_heads == 1 (one weight for all heads) and h' = h when proj_heads == Hq.  It
 *     applies to rows with no marginal block too (O_linear = 0 there, so they get b_h).
 *     O_linear and W are rounded to bf16 for the matrix-core product (fp32 accumulation).
 *   Rows t >= n_valid are written as 0.
 * lse (nullable, fp32 [B, Hq, N]): for training, the natural log-sum-exp of each row's
 *   sparse-branch logits, ln sum_s exp(scale q_t . k_s) over the allowed keys (-inf for a row
 *   with none and for rows t >= n_valid); sla_attn_bwd reads it.
 * q: [B, Hq, N, d]; k, v: [B, Hkv, N, d]; all the same dtype.  out: contiguous
 * [B, Hq, N, d] in out_dtype (SLA_BF16 or SLA_F32).  The linear branch needs causal == 0.
 * Arithmetic: bf16 matrix-core products (fp32 inputs are rounded to bf16), fp32
 * softmax statistics and accumulators.
 * workspace: sla_attn_workspace_bytes(B, Hs, nqb, d, lin_mode) bytes (0 unless MARGINAL).
 */
sla_status sla_attn_fwd(const sla_tensor* q, const sla_tensor* k, const sla_tensor* v, int32_t n_valid,
                        float scale, int32_t causal, int32_t window_tokens, int32_t group_map,
                        const int32_t* crit_rowptr, const int32_t* crit_idx, const uint8_t* crit_flags,
                        const uint32_t* marg_bits,
                        int32_t lin_mode, const void* H, const float* z,
                        const float* H_all, const float* z_all, const float* w_gate,
                        const float* proj_w, const float* proj_b, int32_t proj_heads,
                        void* out, int32_t out_dtype, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Token order along a 3-D Hilbert curve ("2025稀疏注意力架构综述", section 11 SpargeAttn: reordering
 * tokens along a Hilbert curve makes the tokens of a block more alike, raising the predicted
 * sparsity).  For a T x H x W latent grid whose tokens are stored row-major (index (t H + h) W + w),
 * order[n] = the row-major index of the n-th token along the curve: cells sorted by their Hilbert
 * index on the cube of side 2^b >= max(T, H, W) (Skilling's transform, coordinates (t, h, w)).
 * Host-only: `order` is a HOST array of T * H * W int32.  SLA_ERR_SHAPE unless T, H, W >= 1;
 * SLA_ERR_RANGE if T H W > 2^31 - 1 or a side exceeds 2^21.
 */
sla_status sla_hilbert_order(int32_t T, int32_t H, int32_t W, int32_t* order);

/*
 * Apply (inverse == 0) or undo (inverse != 0) a token order on the rows of x [B, H, N, d]:
 *   gather:  out[b,h,n,:] = x[b,h,order[n],:]   for n < n_order,
 *   scatter: out[b,h,order[n],:] = x[b,h,n,:]   for n < n_order,
 * rows n >= n_order are copied unchanged (padding stays at the end).  order: DEVICE int32
 * [n_order], a permutation of 0 .. n_order - 1 (an entry out of range leaves its row in place;
 * with repeated entries the scatter result is unspecified).  out: contiguous [B, H, N, d] in x's
 * dtype, 16-byte aligned, not x itself.  n_order <= N.  A row copy: 2 N d (bf16: 2 bytes) bytes
 * per head moved.  workspace: none.
 */
sla_status sla_permute_rows(const sla_tensor* x, const int32_t* order, int32_t n_order, int32_t inverse,
                            void* out, void* stream);

/* Workspace bytes sla_nsa3_fwd needs (0 for unsupported arguments). */
size_t sla_nsa3_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t d, int32_t dtype,
                                int32_t n_valid, int32_t window_tokens, int32_t cmp_block, int32_t cmp_stride);

/*
 * NSA with its three parallel branches ("Sparse Attention 方法综述", section 2 NSA: compressed,
 * selected and sliding-window branches merged; key parameters: compression block 32 with stride
 * 16, 16 selected blocks of 64, a 512-token window).  For query row t of head h (KV head g):
 *   compressed: softmax attention over compressed tokens m, each the mean of K (and V) rows
 *               m * cmp_stride .. m * cmp_stride + cmp_block - 1 (windows inside the valid rows),
 *               visible when m * cmp_stride + cmp_block - 1 <= t;
 *   selected:   softmax attention over keys s <= t of the blocks in the selection map (the
 *               causal map sla_block_map writes with window_tokens = 0 from group-summed scores);
 *   window:     softmax attention over keys 0 <= t - s < window_tokens;
 *   O[t] = sum over the branches b = (compressed, selected, window) of
 *          sigmoid(q_t . w_gates[b, h]) * O_b[t]   (w_gates: fp32 [3, Hq, d]; an empty branch is 0).
 * Rows t >= n_valid are written as 0.  q [B, Hq, N, d], k, v [B, Hkv, N, d], one dtype; out
 * contiguous [B, Hq, N, d] in out_dtype.  Arithmetic as sla_attn_fwd (bf16 matrix-core products,
 * fp32 statistics); compressed tokens are fp32 means stored in the input dtype.
 * workspace: sla_nsa3_workspace_bytes(...) bytes (compressed K/V, block lists, three fp32 outputs).
 */
sla_status sla_nsa3_fwd(const sla_tensor* q, const sla_tensor* k, const sla_tensor* v, int32_t n_valid,
                        float scale, const int32_t* sel_rowptr, const int32_t* sel_idx, const uint8_t* sel_flags,
                        int32_t window_tokens, int32_t cmp_block, int32_t cmp_stride, const float* w_gates,
                        void* out, int32_t out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes sla_attn_bwd needs (0 for unsupported sizes); proj_heads as passed to
 * sla_attn_bwd (0 without Proj: the Proj buffers are then left out). */
size_t sla_attn_bwd_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t d, int32_t proj_heads);

/*
 * Backward of the SLA layer (the method is fine-tuned: SLA analysis page for arXiv
 * 2509.24006, the learned Proj and linear path).  Gradients of sum(dout * O) with respect to
 * Q, K, V (and the Proj weight and bias), where O is the sla_attn_fwd output in SLA mode, for
 * the SAME block map (held fixed: it is piecewise constant in Q and K):
 *   critical branch:  P = exp(scale q.k - lse), dP = dO V^T, D_t = dO_t . O_sparse_t,
 *                     dS = P (dP - D); dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO;
 *   marginal branch:  through O_linear[t] = phi(q_t)^T S_r / (phi(q_t) . u_r), S_r and u_r the
 *                     sums of H_j = phi(K_j)^T V_j and z_j over row r's marginal blocks;
 *   Proj (proj_w non-NULL): O = O_sparse + W_h O_linear + b_h on valid rows, so the gradient
 *                     reaching O_linear is W_h^T dO, dW_h = sum_t dO_t O_linear_t^T and
 *                     db_h = sum_t dO_t over the valid rows (summed over the heads and
 *                     sequences that share the weight when proj_heads == 1);
 *   smooth-K (k_shift non-NULL): the linear branch used K - mean(K) (mean over the valid rows);
 *                     its key gradient G is evaluated at the shifted keys and becomes
 *                     G - mean over valid rows of G, the path through the mean.
 * Inputs: q, k, v and o (the forward output), dout: [B, H, N, d], one dtype (bf16 or fp32),
 * one KV head per query head (Hq == Hkv, else SLA_ERR_UNSUPPORTED); lse [B, H, N] from
 * sla_attn_fwd; the block map's critical CSR lists and marginal bit masks; S (bf16 bits
 * [rows, d, d]) and u (fp32 [rows, d]) as written by sla_marginal_states for that map (from
 * the shifted keys' states under smooth-K).  k_shift: fp32 [B, H, d] (16-byte aligned) as
 * given to the forward's sla_linear_kv_reduce, or NULL.  proj_w, proj_b, proj_heads: as given
 * to sla_attn_fwd (NULL, NULL, any: no Proj).
 * Outputs dq, dk, dv: contiguous fp32 [B, H, N, d], 16-byte aligned, fully overwritten; rows
 * t >= n_valid are zero.  dproj_w (required with Proj, else NULL): fp32 [proj_heads, d, d],
 * fully overwritten; dproj_b (nullable; NULL without Proj): fp32 [proj_heads, d].
 * O_sparse is taken as o - Proj(O_linear), and D is formed from dO as the matrix-core products
 * see it (rounded to bf16 for fp32 inputs), so dP - D cancels exactly where a row's softmax is
 * constant; with a bf16 o the rounding of the stored sum O_sparse + O_linear stays in D.
 * Arithmetic: bf16 matrix-core operands (the Proj weight rounded to bf16), fp32 accumulation;
 * deterministic (no atomics on gradients).
 * Errors: SLA_ERR_NULL for a missing required pointer or a Proj output without proj_w,
 * SLA_ERR_SHAPE for proj_heads not 1 or H, SLA_ERR_ALIGN, SLA_ERR_WORKSPACE.
 * workspace: sla_attn_bwd_workspace_bytes(B, H, N, d, proj_w ? proj_heads : 0) bytes.
 */
sla_status sla_attn_bwd(const sla_tensor* q, const sla_tensor* k, const sla_tensor* v,
                        const sla_tensor* o, const sla_tensor* dout, const float* lse, int32_t n_valid,
                        float scale, const int32_t* crit_rowptr, const int32_t* crit_idx,
                        const uint32_t* marg_bits, const void* S, const float* u, const float* k_shift,
                        const float* proj_w, const float* proj_b, int32_t proj_heads,
                        float* dq, float* dk, float* dv, float* dproj_w, float* dproj_b,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes sla_attn_bwd_ext needs for these shapes and options (0 for unsupported ones);
 * proj_heads 0 without Proj. */
size_t sla_attn_bwd_ext_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t d,
                                        int32_t lin_mode, int32_t causal, int32_t group_map,
                                        int32_t proj_heads);

/*
 * Backward of every sla_attn_fwd mode for a fixed block map: gradients of sum(dout * O) with
 * respect to Q, K, V and the learned parameters of the mode.  The pages fine-tune both hybrids
 * (SLA analysis page for arXiv 2509.24006: Proj and the linear path; SALAD page, method
 * framework: the gated linear branch) and NSA trains its selection end to end ("Sparse
 * Attention 方法综述", section 2 NSA), so each forward has its backward.  With P, dP, D and dS as
 * in sla_attn_bwd over each row's ALLOWED keys (the forward's masks), per lin_mode:
 *   SLA_LIN_ROW_STATES (MARGINAL maps; S, u and marg_bits as for sla_attn_bwd): the marginal
 *     branch, Proj (proj_w, proj_b, proj_heads, dproj_w, dproj_b) and smooth-K as sla_attn_bwd;
 *   SLA_LIN_GLOBAL_GATED (H_all, z_all fp32 from sla_linear_kv_reduce, w_gate [Hq, d] fp32):
 *     O_linear = g y with g = sigmoid(q . w_gate[h]) and y = phi(q)^T H_all / (phi(q) . z_all):
 *     the gradient reaching y is g dO; dlogit = g (1 - g) (dO . y) adds dlogit w_gate[h] to dq
 *     and dw_gate[h] = sum over b and valid rows of dlogit q (dw_gate fp32 [Hq, d], required);
 *     dH_all, dz_all are the sums over every query block of the per-block state gradients;
 *     smooth-K as above;
 *   SLA_LIN_NONE: the sparse branch alone (D = dout . o); with causal != 0 the forward's causal
 *     masks (s <= t, and flag bit 0 of the entry or t - s < window_tokens; crit_flags required).
 * GQA: q, o, dout [B, Hq, N, d]; k, v [B, Hkv, N, d], Hq a multiple of Hkv, query head h reads
 * KV head h / (Hq / Hkv); dk, dv sum over the query heads of each KV head.  group_map != 0: the
 * map rows are per KV head (Hs = Hkv, as sla_block_map wrote them from group-summed scores), else
 * per query head.  A linear branch needs causal == 0 and group_map == 0 (SLA_ERR_UNSUPPORTED);
 * Proj needs SLA_LIN_ROW_STATES; k_shift (fp32 [B, Hkv, d]) needs a linear branch.
 * lse: fp32 [B, Hq, N] written by the forward.  Outputs dq [B, Hq, N, d], dk, dv [B, Hkv, N, d]
 * contiguous fp32, 16-byte aligned, fully overwritten (rows >= n_valid zero); pointers a mode
 * does not use must be NULL for the outputs (dw_gate, dproj_w, dproj_b) and are ignored for the
 * inputs.  Arithmetic, determinism and error codes as sla_attn_bwd.
 * workspace: sla_attn_bwd_ext_workspace_bytes(B, Hq, Hkv, N, d, lin_mode, causal, group_map,
 * proj_w ? proj_heads : 0) bytes.
 */
sla_status sla_attn_bwd_ext(const sla_tensor* q, const sla_tensor* k, const sla_tensor* v,
                            const sla_tensor* o, const sla_tensor* dout, const float* lse, int32_t n_valid,
                            float scale, int32_t lin_mode, int32_t causal, int32_t window_tokens,
                            int32_t group_map, const int32_t* crit_rowptr, const int32_t* crit_idx,
                            const uint8_t* crit_flags, const uint32_t* marg_bits, const void* S,
                            const float* u, const float* H_all, const float* z_all, const float* w_gate,
                            const float* k_shift, const float* proj_w, const float* proj_b,
                            int32_t proj_heads, float* dq, float* dk, float* dv, float* dproj_w,
                            float* dproj_b, float* dw_gate, void* workspace, size_t workspace_bytes,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SLA_H */
