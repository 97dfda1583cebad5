/*
 * mcs.h — C ABI of libmcs: Meta-Cached Sparse Attention (MC-Sparse) on one
 * AMD Instinct MI355X (gfx950).
 *
 * The method (abstract of "MC-Sparse: Deconstructing and Closing the
 * Dense-Sparse Attention Gap in Diffusion Transformers"; the section
 * "MC-Sparse: three failure modes, one fix" of "The quality cliff nobody
 * admits to"; the three design choices listed in "MC-Sparse Narrows the
 * Dense-Sparse Attention Gap in Diffusion Transformers") has two stages:
 *
 *   selection  exact dense attention; queries are organised into groups of
 *              similar queries that fill whole GPU tiles; each group keeps the
 *              individual KV tokens that carry the most exact attention
 *              probability; the query groups, the kept KV indices and the
 *              difference O_dense - O_sparse of the step's outputs are cached;
 *   reuse      on later denoising steps, attention of each group over only its
 *              cached KV tokens, plus the cached residual.
 *
 * Readings where the pages give no formula: the grouping key is an 8-bit sign
 * hash of each query against 8 caller-supplied projections (bit b set iff the
 * float64 dot product q . r_b, accumulated in dimension order, is > 0); the
 * tokens are stably sorted by key and cut into groups of G consecutive sorted
 * tokens (the last group may be shorter); a group scores key j by the sum of
 * its queries' exact probabilities P_ij; it keeps the k_h best keys (ties to
 * the lower index, compared as float32), stored in ascending order; the sparse
 * softmax is renormalised over the kept keys; the residual O_dense - O_sparse
 * is kept in float32 and added back unchanged on every reuse step.
 *
 * Conventions for every call:
 *  - Tensors Q, K, V, O are [H][N][d] row-major (d contiguous) in the
 *    descriptor's dtype, in device memory, 16-byte aligned.  Batch is folded
 *    into H.
 *  - All calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Results are valid once the stream reaches the call.  No call
 *    synchronises the device, except in the debug mode: with the environment
 *    variable MCS_DEBUG set to a value other than 0 when the library first
 *    launches, every launch is followed by a synchronisation of the stream
 *    and a status check, so that a fault is returned (MCS_ERROR_HIP) by the
 *    call whose kernel caused it.  That mode is not for graph capture.  The device work of every call is kernel
 *    launches only (no allocation, memset or copy; host tables travel as
 *    kernel arguments), so a call can be captured in a HIP graph and
 *    replayed; a replay reads the buffers and host values of the capture.
 *  - The caller owns every device buffer.  The library allocates no device
 *    memory and keeps no global state apart from a per-thread last HIP error.
 *  - Every argument is validated before anything is launched; a call that
 *    returns an error status has not written any output.
 *  - H == 0 or N == 0 is a valid empty problem: the call validates, fills any
 *    host-side output struct and returns MCS_SUCCESS without launching.
 *  - The functions are re-entrant; calls that share output buffers on
 *    different streams race.
 *  - Inputs are expected to be finite.  A NaN or infinity in Q, K or V
 *    gives unspecified values in the outputs that depend on it (never an
 *    access outside the buffers); the bf16 kernels are compiled on the
 *    assumption that no NaN arises.
 */
#ifndef MCS_H_
#define MCS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MCS_VERSION 3
#define MCS_META_VERSION 3
#define MCS_HASH_BITS 8
#define MCS_MAX_SEQ_LEN (1 << 22)

typedef enum mcs_status {
  MCS_SUCCESS = 0,
  MCS_ERROR_INVALID_VALUE = 1,    /* null pointer, negative size, keep outside [1, N] */
  MCS_ERROR_UNSUPPORTED_SHAPE = 2,/* head_dim not 64/128, group not 64/128, dtype unknown, N too large */
  MCS_ERROR_MISALIGNED = 3,       /* a device pointer is not 16-byte (tensors) / 256-byte (meta, workspace) aligned */
  MCS_ERROR_BUFFER_TOO_SMALL = 4, /* meta buffer or workspace smaller than required */
  MCS_ERROR_META_MISMATCH = 5,    /* metadata built for another shape, dtype or layout version */
  MCS_ERROR_HIP = 6               /* a HIP runtime call or launch failed; see mcs_last_hip_error() */
} mcs_status;

typedef enum mcs_dtype {
  MCS_DTYPE_FP32 = 0,  /* float32 in and out; float32 arithmetic */
  MCS_DTYPE_BF16 = 1   /* bfloat16 in and out; bf16 matrix products with float32 accumulation (the
                          selection's P.V products: float16, with each head's V rounded to float16
                          once per selection, scaled by a power of two when it exceeds float16's
                          range) */
} mcs_dtype;

/* Shape of one attention layer. */
typedef struct mcs_attn_desc {
  int32_t num_heads;     /* H >= 0 */
  int32_t seq_len;       /* N, 0 <= N <= MCS_MAX_SEQ_LEN */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t dtype;         /* mcs_dtype */
  float softmax_scale;   /* logits are scale * q.k; a value <= 0 selects 1/sqrt(d) */
} mcs_attn_desc;

/*
 * Cached metadata of one selection step: a value struct describing regions of
 * a caller-owned device buffer (`base`).  The layout is public so that it can
 * be saved, restored or filled by other code.  All offsets are in bytes from
 * `base` and 256-byte aligned.
 *
 *   perm      int32 [H][N]     perm[h][p] = original token at sorted position p;
 *                              group g of head h is positions [g*G, min(N,(g+1)*G))
 *   keep      int32 [H]        k_h, the kept-key budget (index slots) per group of
 *                              head h, 1 <= k_h <= N
 *   idx_start int64 [H]        element offset of head h's indices in `idx`
 *   sched     int32 [H]        heads by decreasing k_h (ties: lower head first);
 *                              reuse launches the costliest heads first
 *   count     int32 [H][ng]    keys kept by group g of head h, 1 <= count <= k_h
 *                              (k_h unless a retained-mass target chose fewer)
 *   order     int32 [H][ng]    launch order of head h's groups in the sparse
 *                              passes: work item t computes group order[h][t].
 *                              Results do not depend on it, but it must be a
 *                              permutation of [0, ng) (a group left out is not
 *                              written).  For hash groups the selection
 *                              writes the groups stably sorted by
 *                              floor(m * 256 / N), m the group's median kept
 *                              key (entry count / 2 of its ascending list), so
 *                              that groups whose kept keys lie in the same part
 *                              of the sequence run side by side and share the
 *                              L2; raster and Z-curve groups, already in
 *                              sequence order, and mcs_meta_init get
 *                              0, 1, ..., ng - 1
 *   idx       int32 [total_idx] head h, group g: the slot of k_h indices at
 *                              idx[idx_start[h] + g*k_h ...]; its first count[h][g]
 *                              entries are the kept keys, ascending
 *   residual  [H][N][d]        O_dense - O_sparse of the selection step, row p
 *                              = sorted position p (not the original token), in
 *                              float32 or (residual_dtype MCS_DTYPE_BF16) bfloat16
 */
typedef struct mcs_meta {
  int32_t version;         /* MCS_META_VERSION */
  int32_t num_heads;
  int32_t seq_len;
  int32_t head_dim;
  int32_t dtype;
  int32_t group_size;      /* G */
  int32_t num_groups;      /* ceil(N / G) */
  int32_t max_keep;        /* max_h k_h */
  int32_t residual_dtype;  /* mcs_dtype of the residual region */
  int32_t reserved;        /* 0 */
  int64_t total_idx;       /* sum_h num_groups * k_h */
  void* base;              /* device pointer to the metadata buffer (NULL from mcs_meta_layout) */
  uint64_t bytes;          /* bytes the layout occupies from base */
  uint64_t off_perm;
  uint64_t off_keep;
  uint64_t off_idx_start;
  uint64_t off_sched;
  uint64_t off_count;
  uint64_t off_order;
  uint64_t off_idx;
  uint64_t off_residual;
} mcs_meta;

/* Library version (MCS_VERSION). */
int mcs_version(void);

/* Static, human-readable name of a status code. */
const char* mcs_status_string(mcs_status status);

/* The hipError_t of the last MCS_ERROR_HIP returned on this thread (0 if none). */
int mcs_last_hip_error(void);

/*
 * Exact dense attention, the method's selection-time computation and the
 * speed baseline every sparse speedup is measured against (the abstract of
 * "MC-Sparse: Deconstructing and Closing the Dense-Sparse Attention Gap in
 * Diffusion Transformers" states its speedups against dense attention).
 *   o[h][i] = sum_j softmax_j(scale * q[h][i] . k[h][j]) v[h][j]
 * q, k, v: [H][N][d] inputs; o: [H][N][d] output (must not alias the inputs).
 */
mcs_status mcs_dense_attn(const mcs_attn_desc* desc, const void* q, const void* k, const void* v,
                          void* o, void* stream);

/*
 * The selection's per-group top-k on caller score rows (the "Individual KV
 * selection" item of "MC-Sparse Narrows the Dense-Sparse Attention Gap in
 * Diffusion Transformers": each group keeps the single KV tokens with the
 * highest scores; mcs_select runs the same kernel on the group key scores it
 * computes).  For each row r < rows of n float32 scores at scores + r * ld,
 * writes the indices of its k largest scores, ties to the lower index, in
 * ascending order to idx[r * k .. r * k + k - 1].  Scores are ranked by their
 * bit patterns as unsigned integers, which is the value order for
 * non-negative floats (the selection's scores are sums of probabilities);
 * other patterns give k distinct indices in that order.  The result is exact
 * for every input: it does not depend on how the rows are read.
 *   scores  device, 16-byte aligned; ld a multiple of 4 with n <= ld; the
 *           buffer holds (rows - 1) * ld + n floats rounded up to a multiple
 *           of 4 (the kernel reads whole 16-byte chunks)
 *   idx     device int32 [rows][k], 4-byte aligned, must not alias scores
 *   n in [1, MCS_MAX_SEQ_LEN], k in [1, n], rows in [0, 2^31 - 1]
 * Errors: MCS_ERROR_INVALID_VALUE for a size or stride outside these
 * ranges or a NULL buffer, MCS_ERROR_MISALIGNED for misaligned buffers.
 */
mcs_status mcs_topk_rows(const float* scores, int64_t ld, int64_t rows, int32_t n, int32_t k, int32_t* idx,
                         void* stream);

/*
 * Host-only: computes the metadata layout (the cached query groups, kept KV
 * indices and residual that the abstract of "MC-Sparse: Deconstructing and
 * Closing the Dense-Sparse Attention Gap in Diffusion Transformers" names)
 * for group size G and per-head keep budgets keep_host[H] (read during the
 * call).  Fills *layout with base = NULL.  Errors as for mcs_select's
 * validation of the same arguments.
 */
mcs_status mcs_meta_layout(const mcs_attn_desc* desc, int32_t group_size, const int32_t* keep_host,
                           mcs_meta* layout);

/* Bytes of metadata buffer that mcs_select needs for the cached groups, kept
 * indices and residual of the abstract of "MC-Sparse: Deconstructing and
 * Closing the Dense-Sparse Attention Gap in Diffusion Transformers" (0 if the
 * arguments are invalid). */
size_t mcs_meta_bytes(const mcs_attn_desc* desc, int32_t group_size, const int32_t* keep_host);

/*
 * mcs_meta_layout for a residual kept in residual_dtype (MCS_DTYPE_FP32, or
 * MCS_DTYPE_BF16 for bf16 problems: half the residual region, the largest
 * part of the metadata cache that the pages count as the method's extra cost,
 * section "MC-Sparse: three failure modes, one fix" of "The quality cliff
 * nobody admits to").  Other residual_dtype values, or BF16 for a float32
 * problem, give MCS_ERROR_INVALID_VALUE.
 */
mcs_status mcs_meta_layout_ex(const mcs_attn_desc* desc, int32_t group_size, const int32_t* keep_host,
                              int32_t residual_dtype, mcs_meta* layout);

/*
 * Bytes of workspace mcs_select needs to process `heads_per_chunk` heads at a
 * time (clamped to [1, H]; 0 if the arguments are invalid).  The bulk is the
 * per-group key scores of the selection (each group's exact probability mass
 * per key: abstract of "MC-Sparse: Deconstructing and Closing the
 * Dense-Sparse Attention Gap in Diffusion Transformers"), float32
 * [heads_per_chunk][ceil(N/G)][N rounded up to 64], plus 64-key block scores
 * (1/64 of that) for block-granular selection, the rows' log-sum-exp
 * (float32 [heads_per_chunk][N]) that the dense pass hands to the key-score
 * pass, and for bf16 problems the chunk's V rounded to float16
 * ([heads_per_chunk][N][d], two bytes each, and two words per head) for the
 * selection's P.V products.  A fixed part holds the grouping's scratch: one
 * key byte and one byte of undecided key bits per token (the hash decides
 * most bits in float32 and recomputes the rest in float64), the stable
 * sort's per-chunk key counts (1 KB per head per 4096 tokens), and the
 * projection tables.
 */
size_t mcs_select_workspace_bytes(const mcs_attn_desc* desc, int32_t group_size, int32_t heads_per_chunk);

struct mcs_select_options; /* defined below */

/* mcs_select_workspace_bytes for a selection with `options` (NULL = the
 * defaults): a bf16 residual adds each head's float32 dense output (float32
 * [heads_per_chunk][N][d]), from which the residual is formed before it is
 * rounded.  0 if the arguments or options are invalid. */
size_t mcs_select_workspace_bytes_ex(const mcs_attn_desc* desc, int32_t group_size, int32_t heads_per_chunk,
                                     const struct mcs_select_options* options);

/*
 * Lays out metadata in meta_buf (device, 256-byte aligned, meta_bytes long)
 * and writes its keep, idx_start and sched regions, every group's count
 * (k_h) and the launch order 0, 1, ..., ng - 1; perm, idx and residual are
 * left for the caller to fill (to restore saved metadata or to supply
 * metadata built elsewhere).  *meta_out receives the descriptor.
 */
mcs_status mcs_meta_init(const mcs_attn_desc* desc, int32_t group_size, const int32_t* keep_host,
                         void* meta_buf, size_t meta_bytes, mcs_meta* meta_out, void* stream);

/* mcs_meta_init for a residual kept in residual_dtype (as mcs_meta_layout_ex).
 * Both write the count region with k_h for every group. */
mcs_status mcs_meta_init_ex(const mcs_attn_desc* desc, int32_t group_size, const int32_t* keep_host,
                            int32_t residual_dtype, void* meta_buf, size_t meta_bytes, mcs_meta* meta_out,
                            void* stream);

/*
 * Selection step (abstract of "MC-Sparse: Deconstructing and Closing the
 * Dense-Sparse Attention Gap in Diffusion Transformers"): groups similar
 * queries into tile-aligned groups, keeps for each group the individual KV
 * tokens that the exact attention probabilities rank highest, and caches the
 * groups, the kept indices and the dense-minus-sparse output difference.
 *   q, k, v        [H][N][d] step inputs (device)
 *   group_size     G, 64 or 128 (query rows per group = one GPU tile)
 *   keep_host      int32 [H] host array, k_h in [1, N], read during the call
 *   hash_proj_host float32 [MCS_HASH_BITS][d] host array of projection
 *                  directions, read during the call
 *   meta_buf       device buffer of meta_bytes >= mcs_meta_bytes(...), 256-aligned
 *   workspace      device buffer of ws_bytes >= mcs_select_workspace_bytes(desc, G, 1),
 *                  256-aligned; more space lets more heads run per chunk
 *   o_dense_out    optional [H][N][d] output (NULL to skip): the exact dense
 *                  output of this step in the original token order
 *   meta_out       host struct receiving the metadata descriptor
 * On success the metadata is complete once the stream reaches the call.
 */
mcs_status mcs_select(const mcs_attn_desc* desc, const void* q, const void* k, const void* v,
                      int32_t group_size, const int32_t* keep_host, const float* hash_proj_host,
                      void* meta_buf, size_t meta_bytes, void* workspace, size_t ws_bytes,
                      void* o_dense_out, mcs_meta* meta_out, void* stream);

/*
 * Ablations of the three failure modes the pages trace the dense-sparse gap
 * to (abstract of "MC-Sparse: Deconstructing and Closing the Dense-Sparse
 * Attention Gap in Diffusion Transformers", and the list in section
 * "MC-Sparse: three failure modes, one fix" of "The quality cliff nobody
 * admits to"): groups that force one pattern on unlike queries, a selection
 * that misjudges which interactions matter, and the attention mass of the
 * dropped tokens.  Each field swaps one of MC-Sparse's
 * choices for the coarser one; all zero-initialised fields but kv_block and
 * residual select MC-Sparse itself.  Two further groupings order the queries
 * differently: the centred hash, and the Z-curve over the latent grid.
 */
typedef enum mcs_grouping {
  MCS_GROUPING_HASH = 0,          /* 8-bit sign hash + stable sort (MC-Sparse) */
  MCS_GROUPING_RASTER = 1,        /* runs of G tokens in raster order (perm = identity) */
  MCS_GROUPING_CENTRED_HASH = 2,  /* sign hash of q_i - mean_i' q_i' (per head; float64 sums in token
                                     order, each product and addition rounded separately) + stable sort */
  MCS_GROUPING_MORTON = 3         /* the tokens, a raster-ordered (T, Y, X) latent grid with token
                                     (t*Y + y)*X + x, in Z-curve order (bits of x, y, t interleaved, x
                                     lowest): a group of 64 is a 4x4x4 block of the grid */
} mcs_grouping;

typedef struct mcs_select_options {
  int32_t grouping;  /* mcs_grouping */
  int32_t kv_block;  /* 1: individual KV tokens (MC-Sparse); 64: whole runs of 64 keys, ranked by the
                        sum of the group's key scores over the run; needs N and every k_h to be
                        multiples of 64 (else MCS_ERROR_UNSUPPORTED_SHAPE) */
  int32_t residual;  /* 1: cache O_dense - O_sparse (MC-Sparse); 0: cache zeros, so reuse returns the
                        sparse output renormalised over the kept keys alone */
  int32_t grid_t, grid_y, grid_x;  /* MCS_GROUPING_MORTON: the latent grid, each in [1, 1024], product at
                                      most N; tokens from the product on (the text tokens of a joint
                                      video + text sequence) follow the grid's tokens in index order;
                                      0 for every other grouping */
  /* Extensions of the method (zero selects the method as read):
     residual_dtype  MCS_DTYPE_FP32 or, for bf16 problems, MCS_DTYPE_BF16: the cached residual
                     O_dense - O_sparse rounded to bfloat16 (computed in float32), half the cache;
                     the metadata buffer is then laid out by mcs_meta_layout_ex with that dtype,
                     and the workspace by mcs_select_workspace_bytes_ex with these options;
     keep_mass       0, or a retained-mass target in (0, 1]: each group keeps the fewest keys, in
                     the top-k order of its scores, whose scores sum to at least keep_mass * |g|
                     (its queries' probability mass: every query's probabilities sum to 1), at
                     most k_h and at least 1; the sum is decided on the float32 scores as
                     fixed-point integers of 2^-48 (floor) against ceil(keep_mass * |g| * 2^48).
                     Needs kv_block 1. */
  int32_t residual_dtype;
  float keep_mass;
  /* Tracing (no effect on the results): NULL, or an array of num_phase_events (0 to
     MCS_SELECT_PHASES) hipEvent_t handles created by the caller on the device of the call.  Event i
     is recorded on the stream when phase i of the selection has been launched: 0 grouping (hash and
     sort, or the fixed order), 1 dense pass, 2 key scores, 3 top-k, 4 residual pass.  When the
     workspace makes the selection run in head chunks, events 1-4 mark the last chunk's phases. */
  void* const* phase_events;
  int32_t num_phase_events;
} mcs_select_options;

#define MCS_SELECT_PHASES 5

/*
 * mcs_select with options (NULL = MC-Sparse: hash groups, single tokens,
 * residual).  Same arguments, ownership and errors as mcs_select; an option
 * outside the values above returns MCS_ERROR_INVALID_VALUE.
 */
mcs_status mcs_select_ex(const mcs_attn_desc* desc, const void* q, const void* k, const void* v,
                         int32_t group_size, const int32_t* keep_host, const float* hash_proj_host,
                         const mcs_select_options* options, void* meta_buf, size_t meta_bytes, void* workspace,
                         size_t ws_bytes, void* o_dense_out, mcs_meta* meta_out, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * mcs_select_ex without a caller workspace.  The workspace is an array of
 * MCS_NOALLOC_SCRATCH_BYTES inside the library, one per device, held from
 * the first use on that device until the process ends.  It must hold the
 * selection's fixed workspace part plus one head's scores, i.e.
 * mcs_select_workspace_bytes(desc, group_size, 1) <= MCS_NOALLOC_SCRATCH_BYTES
 * (else MCS_ERROR_BUFFER_TOO_SMALL, before any other check or launch); the
 * heads then run in as many chunks as the array needs.  Every other argument,
 * result and error is as for mcs_select_ex.  All calls on one device share
 * the array: calls that overlap on one device (on different streams, or
 * from different threads without ordering) race.  Nothing in the array
 * needs to start at zero, so each call may follow any earlier one.
 */
#define MCS_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

mcs_status mcs_select_noalloc(const mcs_attn_desc* desc, const void* q, const void* k, const void* v,
                              int32_t group_size, const int32_t* keep_host, const float* hash_proj_host,
                              const mcs_select_options* options, void* meta_buf, size_t meta_bytes,
                              void* o_dense_out, mcs_meta* meta_out, void* stream);

/*
 * Reuse step (same abstract: the cached groups, indices and residual serve
 * the later denoising steps; the residual restores the attention contribution that renormalising over
 * the kept tokens loses, section "What Trips People Up" of "The quality cliff
 * nobody admits to"):
 *   o[h][perm[p]] = sum_{j in S_g} softmax_{j in S_g}(scale q.k_j) v_j + residual[h][p]
 * for every sorted position p of group g, S_g = the group's cached keys.
 * q, k, v: [H][N][d] inputs of this step; meta: from mcs_select or
 * mcs_meta_init with the same H, N, d and dtype; o: [H][N][d] output.
 * Errors: MCS_ERROR_META_MISMATCH when meta was built for another shape,
 * dtype or layout version, or when its region offsets or size are not the
 * ones this layout gives for its own total_idx.  Edited metadata cannot
 * lead a kernel out of bounds: permutation entries are clamped to [0, N),
 * and kept-key gathers go through bounds-checked buffer loads (an index
 * outside [0, N) reads zeros).
 */
mcs_status mcs_sparse_attn(const mcs_attn_desc* desc, const void* q, const void* k, const void* v,
                           const mcs_meta* meta, void* o, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MCS_H_ */
