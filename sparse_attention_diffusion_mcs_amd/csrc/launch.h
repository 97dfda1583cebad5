// Internal host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mcs {

enum AttnMode : int {
  MODE_PLAIN = 0,    // dense, natural row order, O out
  MODE_SELECT = 1,   // dense over group-sorted rows: O_dense (float32, sorted rows) + row lse (bf16);
                     // the float32 kernel also writes the per-group key scores
  MODE_REUSE = 2,    // sparse over cached keys + residual, O out in original order
  MODE_RESINIT = 3,  // sparse over cached keys at selection: residual -= O_sparse
  MODE_SCORE = 4     // selection key scores from the rows' log-sum-exp (bf16 only)
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* v16;           // SELECT/RESINIT (bf16): V * 2^-v16_exp[head] rounded to float16, [nheads][N][d] of
                             // the launch's heads
  const int* v16_exp;        // SELECT/RESINIT (bf16): per launch head, the power of two V was scaled down by
  void* o;                   // PLAIN/REUSE: output; SELECT: optional dense output (original order)
  void* residual;            // [H][N][d], sorted-position rows: float32, or bf16 when residual_bf16
  int residual_bf16;         // REUSE/RESINIT: the residual region holds bf16
  float* odense;             // SELECT out, RESINIT in: float32 dense output [nheads][N][d] (sorted rows), when
                             // the residual is bf16 (else SELECT writes it into the float32 residual region)
  const int32_t* count;      // [H][ng] kept keys per group (REUSE, RESINIT)
  const int32_t* order;      // [H][ng] launch order of the groups (REUSE, RESINIT; null: index order)
  float keep_mass;           // selection: retained-mass target (0: fixed budgets)
  float* colsum;             // SCORE: [nheads][ng][ldc] key scores of the launched heads
  float* lse;                // SELECT out, SCORE in: [nheads][N] log2-sum-exp of the sorted rows
  const int32_t* perm;       // [H][N]
  const int32_t* keep;       // [H]
  const int64_t* idx_start;  // [H]
  const int32_t* sched;      // [H] (REUSE)
  const int32_t* idx;        // kept keys
  int H, N, D, G, ng, ldc;
  long long total_idx;       // entries in idx (sparse modes; bounds every gather)
  int head0;                 // first head of the launch (PLAIN/SELECT/RESINIT)
  int nheads;                // heads in the launch
  float scale;               // softmax scale
  int run;                   // XCD run length (logical blocks per XCD per round)
  int kchunks;               // SCORE: key ranges per row tile (set at launch)
};

// bf16 MFMA kernels (attn_bf16.hip)
hipError_t launch_attn_bf16(int mode, const AttnArgs& a, hipStream_t s);
// float32 VALU kernels (attn_f32.hip)
hipError_t launch_attn_f32(int mode, const AttnArgs& a, hipStream_t s);

// selection helpers (select.hip)
// proj: the projections as float64 [8][D], then as float32 [8][D], then the
// float32 coefficient of each projection's decision threshold [8];
// mean: per-head query means (float64 [H][D]) for the centred hash, or null;
// undecided: H*N bytes of scratch (the key bits the float32 pass leaves to
// the float64 one)
hipError_t launch_hash_keys(const void* q, int dtype, const double* proj, const double* mean, uint8_t* keys,
                            uint8_t* undecided, int H, int N, int D, hipStream_t s);
hipError_t launch_query_mean(const void* q, int dtype, double* mean, int H, int N, int D, hipStream_t s);
// The bf16 V of nheads heads (per_head values each, a multiple of 8, 16-byte
// aligned) rounded to float16 into out, each head scaled by 2^-vexp[head]:
// 0, or the smallest power of two that brings the head's largest finite
// magnitude within float16's range.  hmax (nheads words) is scratch.
hipError_t launch_v_to_f16(const void* v, void* out, int nheads, long long per_head, uint32_t* hmax, int* vexp,
                           hipStream_t s);
// Stable sort of each head's token keys; counts: H * 256 * sort_chunks(N)
// int32 of scratch
int sort_chunks(int N);
hipError_t launch_perm_sort(const uint8_t* keys, int32_t* perm, int32_t* counts, int H, int N, hipStream_t s);
// Writes each group's kept keys (idx) and their number (count[h][g]); with
// keep_mass > 0 the number comes from the retained-mass target (groups of G
// of the nq queries), else it is keep[h] / block blocks.
hipError_t launch_group_topk(const float* colsum, int ldc, int32_t* idx, int32_t* count, const int32_t* keep,
                             const int64_t* idx_start, int head0, int nheads, int ng, int N, int G, int nq, int block,
                             float keep_mass, hipStream_t s);
// Top-k of `rows` plain score rows (row r at scores + r * ld, n scores; ld a
// multiple of 4, at least n): the k largest of each row, ties to the lower
// index, written ascending to idx + r * k.
hipError_t launch_topk_rows(const float* scores, int ld, int rows, int n, int k, int32_t* idx, hipStream_t s);
// count[h][g] = keep[h] for every group of every head (device tables)
hipError_t launch_fill_counts(int32_t* count, const int32_t* keep, int H, int ng, hipStream_t s);
// Launch order of the groups of heads head0 .. head0+nheads-1 for the sparse
// passes: each group's sort key floor(m * 256 / N), m its median kept key
// (entry count/2 of its ascending list), goes to bucket[h][g] (bytes,
// [H][ng]); order[h] is then the stable order of the keys.
hipError_t launch_group_order(const int32_t* idx, const int32_t* count, const int32_t* keep,
                              const int64_t* idx_start, uint8_t* bucket, int32_t* order, int head0, int nheads, int ng,
                              int N, long long total_idx, hipStream_t s);
// ablation helpers: 64-key block scores of score rows, raster-order
// permutation, zero fill (residual off)
hipError_t launch_block_scores(const float* colsum, int ldc, float* bs, int ldb, long long rows, int nb,
                               hipStream_t s);
hipError_t launch_iota_perm(int32_t* perm, int H, int N, hipStream_t s);
// Z-curve order of a raster-ordered (T, Y, X) grid, N = T * Y * X, every dim <= 1024
hipError_t launch_morton_perm(int32_t* perm, int H, int N, int T, int Y, int X, hipStream_t s);
hipError_t launch_zero_floats(float* p, long long n, hipStream_t s);
// Device address of the current device's MCS_NOALLOC_SCRATCH_BYTES scratch
// array (noalloc.hip), the workspace of mcs_select_noalloc.
hipError_t noalloc_scratch(void** out);
// Writes `nbytes` bytes from host memory to device memory through kernel
// arguments (asynchronous on s, safe for pageable and stack host memory).
hipError_t launch_fill_bytes(void* dst, const void* src, size_t nbytes, hipStream_t s);

// Status of the launch just made on s: the launch error; with MCS_DEBUG set
// to a value other than 0 in the environment, the stream is also synchronised
// and a fault of the kernel is returned here, at the launch that caused it
// (mcs_api.cpp; not for use under graph capture).
hipError_t launched(hipStream_t s);
bool debug_sync();

}  // namespace mcs
