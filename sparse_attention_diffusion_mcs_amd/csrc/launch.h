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
  void* o;                   // PLAIN/REUSE: output; SELECT: optional dense output (original order)
  float* residual;           // [H][N][d], sorted-position rows
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
// mean: per-head query means (float64 [H][D]) for the centred hash, or null
hipError_t launch_hash_keys(const void* q, int dtype, const double* proj, const double* mean, uint8_t* keys, int H,
                            int N, int D, hipStream_t s);
hipError_t launch_query_mean(const void* q, int dtype, double* mean, int H, int N, int D, hipStream_t s);
hipError_t launch_perm_sort(const uint8_t* keys, int32_t* perm, int H, int N, hipStream_t s);
hipError_t launch_group_topk(const float* colsum, int ldc, int32_t* idx, const int32_t* keep,
                             const int64_t* idx_start, int head0, int nheads, int ng, int N, int block,
                             hipStream_t s);
// ablation helpers: 64-key block scores of score rows, raster-order
// permutation, zero fill (residual off)
hipError_t launch_block_scores(const float* colsum, int ldc, float* bs, int ldb, long long rows, int nb,
                               hipStream_t s);
hipError_t launch_iota_perm(int32_t* perm, int H, int N, hipStream_t s);
// Z-curve order of a raster-ordered (T, Y, X) grid, N = T * Y * X, every dim <= 1024
hipError_t launch_morton_perm(int32_t* perm, int H, int N, int T, int Y, int X, hipStream_t s);
hipError_t launch_zero_floats(float* p, long long n, hipStream_t s);
// Writes `nbytes` bytes from host memory to device memory through kernel
// arguments (asynchronous on s, safe for pageable and stack host memory).
hipError_t launch_fill_bytes(void* dst, const void* src, size_t nbytes, hipStream_t s);

}  // namespace mcs
