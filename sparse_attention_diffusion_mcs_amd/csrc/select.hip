// Selection-step helper kernels for gfx950: the query hash, the stable
// group-order permutation and the per-group exact top-k.
//
// Method: abstract of "MC-Sparse: Deconstructing and Closing the Dense-Sparse
// Attention Gap in Diffusion Transformers" (similar queries are organised into
// tile-aligned groups; each group keeps individual KV tokens chosen from exact
// attention probabilities) and the list of design choices in "MC-Sparse
// Narrows the Dense-Sparse Attention Gap in Diffusion Transformers"
// ("Hardware-aware query organization", "Individual KV selection").
//
// Readings: key_i = sum_b [q_i . r_b > 0] 2^b with the dot product accumulated
// in float64 in dimension order (every product of a bf16/float32 input with a
// float32 projection is exact in float64, so the key is a well-defined
// function of the inputs); tokens are stably sorted by key; a group keeps the
// k keys of largest float32 score, ties to the lower key index, ascending.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace mcs {
namespace {

// ---------------------------------------------------------------- hash ----
template <typename T>
__device__ __forceinline__ float load_elem(const T* p);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// With CENTRED the queries are first centred on their head's mean (`mean`,
// float64 [H][D]); each product and each addition is then rounded on its own
// (__dmul_rn, __dadd_rn), because the centred values no longer multiply
// exactly.  Without it every product of a bf16/float32 value and a float32
// projection is exact in float64 and one fused multiply-add per term gives
// the same sum.
template <typename T, int D, bool CENTRED>
__global__ __launch_bounds__(256) void hash_keys_kernel(const T* __restrict__ q, const double* __restrict__ proj,
                                                         const double* __restrict__ mean, uint8_t* __restrict__ keys,
                                                         long long total, int N) {
  __shared__ double r[8][D];
  for (int e = threadIdx.x; e < 8 * D; e += 256) r[e / D][e % D] = proj[e];
  __syncthreads();
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const T* row = q + i * D;
  const double* mu = CENTRED ? mean + (i / N) * D : nullptr;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int c = 0; c < D; ++c) {
    const double x = (double)load_elem<T>(row + c);
    if constexpr (CENTRED) {
      const double xc = x - mu[c];
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[b] = __dadd_rn(acc[b], __dmul_rn(xc, r[b][c]));
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[b] = __fma_rn(x, r[b][c], acc[b]);
    }
  }
  uint32_t key = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) key |= (acc[b] > 0.0 ? 1u : 0u) << b;
  keys[i] = (uint8_t)key;
}

// Per-dimension mean of each head's queries: one thread per (head, dim),
// float64 sums in token order, one division.
template <typename T, int D>
__global__ __launch_bounds__(D) void query_mean_kernel(const T* __restrict__ q, double* __restrict__ mean, int N) {
  const int h = blockIdx.x, c = threadIdx.x;
  const T* col = q + (size_t)h * N * D + c;
  double sum = 0.0;
  int i = 0;
  for (; i + 8 <= N; i += 8) {
    double x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = (double)load_elem<T>(col + (size_t)(i + u) * D);
#pragma unroll
    for (int u = 0; u < 8; ++u) sum = __dadd_rn(sum, x[u]);
  }
  for (; i < N; ++i) sum = __dadd_rn(sum, (double)load_elem<T>(col + (size_t)i * D));
  mean[(size_t)h * D + c] = sum / (double)N;
}

// ---------------------------------------------------------- stable sort ----
// One workgroup per head.  A 256-bin histogram gives each key's first
// position; tokens are then placed tile by tile in token order, with the rank
// among equal keys inside a wave found by ballots over the 8 key bits and
// across the waves of a tile by an ordered prefix over per-wave counts, so the
// result is the stable order.
constexpr int SORT_NT = 1024;
constexpr int SORT_NW = SORT_NT / 64;

__global__ __launch_bounds__(SORT_NT) void perm_sort_kernel(const uint8_t* __restrict__ keys,
                                                            int32_t* __restrict__ perm, int N) {
  __shared__ int hist[256];
  __shared__ int base[256];
  __shared__ int cnt[SORT_NW][256];
  const int h = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const uint8_t* kh = keys + (size_t)h * N;
  int32_t* ph = perm + (size_t)h * N;

  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  for (int i = tid; i < N; i += SORT_NT) atomicAdd(&hist[kh[i]], 1);
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int b = 0; b < 256; ++b) {
      base[b] = run;
      run += hist[b];
    }
  }
  __syncthreads();

  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int t0 = 0; t0 < N; t0 += SORT_NT) {
    for (int e = tid; e < SORT_NW * 256; e += SORT_NT) (&cnt[0][0])[e] = 0;
    __syncthreads();
    const int i = t0 + tid;
    const bool valid = i < N;
    const int key = valid ? kh[i] : 0;
    unsigned long long same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (key >> b) & 1;
      const unsigned long long bb = __ballot(valid && bit);
      same &= bit ? bb : ~bb;
    }
    const int rank = __popcll(same & lt_mask);
    const bool leader = valid && (same >> lane) == 1ull;
    if (leader) cnt[w][key] = __popcll(same);
    __syncthreads();
    if (tid < 256) {
      int r = base[tid];
      for (int ww = 0; ww < SORT_NW; ++ww) {
        const int c = cnt[ww][tid];
        cnt[ww][tid] = r;
        r += c;
      }
      base[tid] = r;
    }
    __syncthreads();
    if (valid) ph[cnt[w][key] + rank] = i;
    __syncthreads();
  }
}

// ---------------------------------------------------------------- top-k ----
// One workgroup per (head, group) score row.  Scores are non-negative floats,
// so their bit patterns order like the values.  Three histogram passes over
// bits [31:21], [20:10], [9:0] find the k-th largest pattern T exactly; a
// final ordered pass writes every index with score > T and the lowest-index
// (k - #greater) indices with score == T, in ascending index order.  When
// the first pass's bin of T holds at most TK_CAP scores, a second read copies
// them into LDS and the last two passes run there: three reads of the row
// instead of four.
constexpr int TK_NT = 256;
constexpr int TK_CAP = 4096;

__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = __lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __builtin_amdgcn_ds_bpermute((lane - off) << 2, x);
    if (lane >= off) x += y;
  }
  return x;
}

// Exclusive block scan of two counters; returns the totals through *ta/*tb.
__device__ __forceinline__ void block_excl_scan2(int a, int b, int* ea, int* eb, int* ta, int* tb, int* sh) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int packed_a = wave_incl_scan(a), packed_b = wave_incl_scan(b);
  if (lane == 63) {
    sh[w] = packed_a;
    sh[4 + w] = packed_b;
  }
  __syncthreads();
  int off_a = 0, off_b = 0, tot_a = 0, tot_b = 0;
#pragma unroll
  for (int ww = 0; ww < TK_NT / 64; ++ww) {
    if (ww < w) {
      off_a += sh[ww];
      off_b += sh[4 + ww];
    }
    tot_a += sh[ww];
    tot_b += sh[4 + ww];
  }
  __syncthreads();
  *ea = off_a + packed_a - a;
  *eb = off_b + packed_b - b;
  *ta = tot_a;
  *tb = tot_b;
}

// One workgroup per (head, group) row of N scores: the keep[h] / block
// largest (ties to the lower index), written ascending.  With block > 1 the
// row holds scores of whole key blocks and every kept block b is written as
// its keys b*block .. b*block + block - 1.
__global__ __launch_bounds__(TK_NT) void group_topk_kernel(const float* __restrict__ colsum, int ldc,
                                                           int32_t* __restrict__ idx, const int32_t* __restrict__ keep,
                                                           const int64_t* __restrict__ idx_start, int head0, int ng,
                                                           int N, int block) {
  __shared__ int hist[2048];
  __shared__ uint32_t cand[TK_CAP];
  __shared__ int sh[8];
  __shared__ int found[3];
  const int tid = threadIdx.x;
  const int g = blockIdx.x, hl = blockIdx.y, h = head0 + hl;
  const uint32_t* row = reinterpret_cast<const uint32_t*>(colsum + ((size_t)hl * ng + g) * ldc);
  const int k = keep[h] / block;
  int32_t* out = idx + idx_start[h] + (int64_t)g * keep[h];

  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  // Reads the row 16 consecutive scores per thread and step (four 16-byte
  // loads in flight; rows start 256-byte aligned) and hands each in-range
  // score to f.
  auto scan_row = [&](auto f) {
    for (int j0 = 16 * tid; j0 < N; j0 += 16 * TK_NT) {
      uint32_t u[16];
      if (j0 + 16 <= N) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 x = *reinterpret_cast<const uint4*>(row + j0 + 4 * v);
          u[4 * v] = x.x;
          u[4 * v + 1] = x.y;
          u[4 * v + 2] = x.z;
          u[4 * v + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) u[e] = (j0 + e < N) ? row[j0 + e] : 0u;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (j0 + e < N) f(u[e]);
    }
  };
  bool in_lds = false;
  int ncand = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int b = tid; b < 2048; b += TK_NT) hist[b] = 0;
    __syncthreads();
    auto count = [&](uint32_t x) {
      if ((x & pmask) == prefix) atomicAdd(&hist[(x >> shift) & (nb - 1)], 1);
    };
    if (in_lds) {
      for (int c = tid; c < ncand; c += TK_NT) count(cand[c]);
    } else {
      scan_row(count);
    }
    __syncthreads();
    // thread t owns bins [t*per, (t+1)*per); `above` = elements in higher bins
    const int per = nb / TK_NT;
    int mine = 0;
    for (int b = 0; b < per; ++b) mine += hist[tid * per + b];
    int excl, unused_e, total, unused_t;
    block_excl_scan2(mine, 0, &excl, &unused_e, &total, &unused_t, sh);
    int above = total - excl - mine;
    if (above < krem && above + mine >= krem) {
      for (int b = per - 1; b >= 0; --b) {
        const int bin = tid * per + b;
        if (above + hist[bin] >= krem) {
          found[0] = bin;
          found[1] = above;
          found[2] = hist[bin];
          break;
        }
        above += hist[bin];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)found[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    krem -= found[1];
    const int in_bin = found[2];
    __syncthreads();
    if (pass == 0 && in_bin <= TK_CAP) {
      // second read: the scores in T's bin, to LDS (exactly in_bin of them)
      if (tid == 0) sh[0] = 0;
      __syncthreads();
      scan_row([&](uint32_t x) {
        if ((x & pmask) == prefix) cand[atomicAdd(&sh[0], 1)] = x;
      });
      __syncthreads();
      ncand = in_bin;
      in_lds = true;
    }
  }
  const uint32_t T = prefix;

  // ordered compaction, 4 consecutive elements per thread per step
  int gt_base = 0, eq_base = 0;
  for (int t0 = 0; t0 < N; t0 += 4 * TK_NT) {
    const int j0 = t0 + 4 * tid;
    uint32_t u[4];
    if (j0 + 4 <= N) {
      const uint4 x = *reinterpret_cast<const uint4*>(row + j0);
      u[0] = x.x;
      u[1] = x.y;
      u[2] = x.z;
      u[3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = (j0 + e < N) ? row[j0 + e] : 0u;
    }
    int ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = j0 + e < N;
      ngt += (in && u[e] > T);
      neq += (in && u[e] == T);
    }
    int pgt, peq, tgt, teq;
    block_excl_scan2(ngt, neq, &pgt, &peq, &tgt, &teq, sh);
    int gt_before = gt_base + pgt, eq_before = eq_base + peq;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (j0 + e >= N) break;
      const bool gt = u[e] > T, eq = u[e] == T;
      const int pos = gt_before + min(eq_before, krem);
      if ((gt || (eq && eq_before < krem)) && pos < k) {
        if (block == 1)
          out[pos] = j0 + e;
        else
          for (int t = 0; t < block; ++t) out[(int64_t)pos * block + t] = (j0 + e) * block + t;
      }
      gt_before += gt;
      eq_before += eq;
    }
    gt_base += tgt;
    eq_base += teq;
  }
}

// ------------------------------------------------ ablation helpers ----
// Score of each run of `block` consecutive keys of a score row (block = 64:
// sixteen float4 reads of one 256-byte run).
__global__ void block_scores_kernel(const float* __restrict__ colsum, int ldc, float* __restrict__ bs, int ldb,
                                    long long rows, int nb) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * nb) return;
  const long long r = i / nb;
  const int b = (int)(i % nb);
  const float4* src = reinterpret_cast<const float4*>(colsum + r * ldc + 64LL * b);
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const float4 x = src[t];
    sum += (x.x + x.y) + (x.z + x.w);
  }
  bs[r * ldb + b] = sum;
}

// Raster-order groups: perm[h][p] = p.
__global__ void iota_perm_kernel(int32_t* __restrict__ perm, long long total, int N) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long long)gridDim.x * blockDim.x)
    perm[i] = (int32_t)(i % N);
}

// Z-curve groups over a raster-ordered (T, Y, X) grid.  A token's Z-curve
// code interleaves the bits of x, y, t (x lowest); its rank among the grid's
// codes is found without sorting: walking the code from the top bit, every
// 1 bit adds the number of grid cells in the lower half of the current
// Z-curve subtree (an axis-aligned box clipped to the grid), then descends
// into the upper half.  perm[h][rank] = token for every head.
__device__ __forceinline__ long long clipped(int lo, int len, int size) {
  return lo >= size ? 0 : (long long)(min(lo + len, size) - lo);
}

__global__ void morton_perm_kernel(int32_t* __restrict__ perm, int H, int N, int T, int Y, int X) {
  const int tok = blockIdx.x * blockDim.x + threadIdx.x;
  if (tok >= N) return;
  const int x = tok % X, y = (tok / X) % Y, t = tok / (X * Y);
  const int size[3] = {X, Y, T}, coord[3] = {x, y, t};
  int lo[3] = {0, 0, 0}, len[3] = {1024, 1024, 1024};
  long long rank = 0;
  for (int p = 29; p >= 0; --p) {
    const int a = p % 3, half = len[a] >> 1;
    if ((coord[a] >> (p / 3)) & 1) {
      long long vol = clipped(lo[a], half, size[a]);
#pragma unroll
      for (int o = 0; o < 3; ++o)
        if (o != a) vol *= clipped(lo[o], len[o], size[o]);
      rank += vol;
      lo[a] += half;
    }
    len[a] = half;
  }
  for (int h = 0; h < H; ++h) perm[(size_t)h * N + rank] = tok;
}

__global__ void zero_floats_kernel(float* __restrict__ p, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// ----------------------------------------------------------- host bytes ----
constexpr int FILL_WORDS = 960;
struct FillPayload {
  uint32_t w[FILL_WORDS];
};

__global__ void fill_words_kernel(uint32_t* dst, FillPayload p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = p.w[i];
}

}  // namespace

namespace {
template <typename T, int D>
void hash_launch(const void* q, const double* proj, const double* mean, uint8_t* keys, long long total, int N,
                 hipStream_t s) {
  const dim3 grid((unsigned)((total + 255) / 256));
  if (mean)
    hipLaunchKernelGGL((hash_keys_kernel<T, D, true>), grid, dim3(256), 0, s, static_cast<const T*>(q), proj, mean,
                       keys, total, N);
  else
    hipLaunchKernelGGL((hash_keys_kernel<T, D, false>), grid, dim3(256), 0, s, static_cast<const T*>(q), proj,
                       mean, keys, total, N);
}
}  // namespace

hipError_t launch_hash_keys(const void* q, int dtype, const double* proj, const double* mean, uint8_t* keys, int H,
                            int N, int D, hipStream_t s) {
  const long long total = (long long)H * N;
  if (total == 0) return hipSuccess;
  if (dtype == 1) {
    if (D == 64)
      hash_launch<uint16_t, 64>(q, proj, mean, keys, total, N, s);
    else
      hash_launch<uint16_t, 128>(q, proj, mean, keys, total, N, s);
  } else {
    if (D == 64)
      hash_launch<float, 64>(q, proj, mean, keys, total, N, s);
    else
      hash_launch<float, 128>(q, proj, mean, keys, total, N, s);
  }
  return hipGetLastError();
}

hipError_t launch_query_mean(const void* q, int dtype, double* mean, int H, int N, int D, hipStream_t s) {
  if (H == 0 || N == 0) return hipSuccess;
  if (dtype == 1) {
    if (D == 64)
      hipLaunchKernelGGL((query_mean_kernel<uint16_t, 64>), dim3(H), dim3(64), 0, s, static_cast<const uint16_t*>(q),
                         mean, N);
    else
      hipLaunchKernelGGL((query_mean_kernel<uint16_t, 128>), dim3(H), dim3(128), 0, s,
                         static_cast<const uint16_t*>(q), mean, N);
  } else {
    if (D == 64)
      hipLaunchKernelGGL((query_mean_kernel<float, 64>), dim3(H), dim3(64), 0, s, static_cast<const float*>(q), mean,
                         N);
    else
      hipLaunchKernelGGL((query_mean_kernel<float, 128>), dim3(H), dim3(128), 0, s, static_cast<const float*>(q),
                         mean, N);
  }
  return hipGetLastError();
}

hipError_t launch_perm_sort(const uint8_t* keys, int32_t* perm, int H, int N, hipStream_t s) {
  if (H == 0 || N == 0) return hipSuccess;
  hipLaunchKernelGGL(perm_sort_kernel, dim3(H), dim3(SORT_NT), 0, s, keys, perm, N);
  return hipGetLastError();
}

hipError_t launch_group_topk(const float* colsum, int ldc, int32_t* idx, const int32_t* keep,
                             const int64_t* idx_start, int head0, int nheads, int ng, int N, int block,
                             hipStream_t s) {
  if (nheads == 0 || ng == 0) return hipSuccess;
  hipLaunchKernelGGL(group_topk_kernel, dim3(ng, nheads), dim3(TK_NT), 0, s, colsum, ldc, idx, keep, idx_start,
                     head0, ng, N, block);
  return hipGetLastError();
}

hipError_t launch_block_scores(const float* colsum, int ldc, float* bs, int ldb, long long rows, int nb,
                               hipStream_t s) {
  const long long total = rows * nb;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(block_scores_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, colsum, ldc, bs,
                     ldb, rows, nb);
  return hipGetLastError();
}

hipError_t launch_iota_perm(int32_t* perm, int H, int N, hipStream_t s) {
  const long long total = (long long)H * N;
  if (total == 0) return hipSuccess;
  const long long blocks = std::min<long long>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(iota_perm_kernel, dim3((unsigned)blocks), dim3(256), 0, s, perm, total, N);
  return hipGetLastError();
}

hipError_t launch_morton_perm(int32_t* perm, int H, int N, int T, int Y, int X, hipStream_t s) {
  if (H == 0 || N == 0) return hipSuccess;
  hipLaunchKernelGGL(morton_perm_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, perm, H, N, T, Y, X);
  return hipGetLastError();
}

hipError_t launch_zero_floats(float* p, long long n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const long long blocks = std::min<long long>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(zero_floats_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_fill_bytes(void* dst, const void* src, size_t nbytes, hipStream_t s) {
  // dst is 4-byte aligned and nbytes a multiple of 4 for every caller
  const uint8_t* in = static_cast<const uint8_t*>(src);
  uint8_t* out = static_cast<uint8_t*>(dst);
  size_t done = 0;
  while (done < nbytes) {
    const size_t chunk = (nbytes - done) < (size_t)FILL_WORDS * 4 ? (nbytes - done) : (size_t)FILL_WORDS * 4;
    FillPayload p;
    __builtin_memcpy(p.w, in + done, chunk);
    hipLaunchKernelGGL(fill_words_kernel, dim3(1), dim3(256), 0, s, reinterpret_cast<uint32_t*>(out + done), p,
                       (int)(chunk / 4));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    done += chunk;
  }
  return hipSuccess;
}

}  // namespace mcs
