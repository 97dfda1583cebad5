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

// The key bit of token i and projection b is [S > 0] for S = q_i . r_b
// accumulated in float64 in dimension order, one fused multiply-add per term
// (every product of a bf16/float32 value and a float32 projection is exact in
// float64).  The kernel first forms S32, the same sum in float32.  With
// A = sum_c |q_ic r_bc| <= |q_i| |r_b| (Cauchy-Schwarz), the two sums of D
// rounded terms are within gamma_D(u) A of the exact sum (the standard bound
// of recursive summation, u = 2^-24 and 2^-53), the float32 one also within
// an absolute D * 2^-126 when results underflow.  So whenever
//   |S32| > (1 + 2^-8) (gamma_D(2^-24) + gamma_D(2^-53)) |r_b| sqrt(|q_i|^2 + 2^-100) + 2^-100
// (the factor 1 + 2^-8 covers the rounding of this threshold, computed in
// float32 from the float32 |q_i|^2, whose own error is at most gamma_D(2^-24)
// relative plus the underflow the 2^-100 term absorbs; the coefficient per
// projection comes from the host, rounded up), the exact sum has the sign of S32 and a magnitude above
// the float64 sum's error, and the float64 sum has the same sign: the bit is
// decided.  The bits left undecided (|S32| below the threshold, or not
// finite) are marked per token, and a second kernel recomputes their sums in
// float64 exactly as defined (hash_fixup_kernel); on Gaussian projections
// about one token in a thousand has such a bit.
//
// With CENTRED the queries are first centred on their head's mean (`mean`,
// float64 [H][D]); each product and each addition is then rounded on its own
// (__dmul_rn, __dadd_rn), because the centred values no longer multiply
// exactly, and the sums are taken in float64 only.
//
// A workgroup of two waves hashes tiles of HR consecutive tokens (rows of the
// flattened [H*N] queries), tile blockIdx.x, then every gridDim.x-th tile
// after it.  Lane r of wave w sums row r of the tile against projections
// 4w .. 4w + 3, in dimension order.  The projection values are then the
// same across the wave and come from scalar loads into SGPRs, batch by batch
// (BD dimensions of four projections): batch m + 1 is loaded while batch m
// is summed.  Scalar loads return out of order, so the wait for a batch
// covers every load in flight, and it comes before the next batch's loads
// are issued; an opaque zero added to each batch's base address keeps the
// compiler from merging the batches' loads or hoisting them out of the tile
// loop (the projections do not fit in SGPRs).  A 64-row tile keeps the LDS per
// workgroup (17.5 KB at d = 128 in bf16) small enough for nine workgroups,
// 18 waves, per CU.  A tile's rows are copied
// with 16-byte buffer loads that consecutive threads issue for consecutive
// addresses, one tile ahead, so the copy overlaps the arithmetic; the
// buffer's range check returns zeros past the last row, so the loads need no
// branches.  The LDS rows are padded by 16 bytes: the row stride in 4-byte
// banks is then odd in units of four banks, so the 16-byte reads of 32 lanes
// of different rows fall into distinct bank groups.  Each wave leaves its
// four key bits in LDS, and the key bytes are written after the barrier
// that ends the tile.
constexpr int HT = 128;  // threads per workgroup: two waves
constexpr int HR = 64;   // rows per tile
constexpr int HASH_BLOCKS_PER_CU = 9;
constexpr int kHashBits = 8;  // projections: two waves of four

template <typename T, int D, bool CENTRED>
__global__ __launch_bounds__(HT) void hash_keys_kernel(const T* __restrict__ q, const double* __restrict__ proj,
                                                        const float* __restrict__ proj32,
                                                        const float* __restrict__ coef,
                                                        const double* __restrict__ mean, uint8_t* __restrict__ keys,
                                                        uint8_t* __restrict__ undecided_out, long long total, int N) {
  constexpr int ROWB = D * (int)sizeof(T);  // bytes per query row
  constexpr int STRIDE = ROWB + 16;         // padded LDS row
  constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per chunk
  constexpr int LPT = HR * CPR / HT;        // 16-byte loads per thread per tile
  constexpr int BD = 4;                     // dimensions per batch
  constexpr int NBAT = D / BD;
  constexpr int BPC = EPC / BD;             // batches per chunk
  static_assert(EPC % BD == 0 && D % EPC == 0, "batches must tile the chunks");
  __shared__ __attribute__((aligned(16))) unsigned char rows[HR * STRIDE];
  __shared__ uint8_t part[2][HR];
  __shared__ uint8_t part_und[2][HR];
  const long long tiles = (total + HR - 1) / HR;
  const unsigned char* base = reinterpret_cast<const unsigned char*>(q);
  const int r = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform

  // chunk e = threadIdx.x + HT * l of tile t: row e / CPR, chunk e % CPR
  auto load_tile = [&](uint4* buf, long long t) __attribute__((always_inline)) {
    const long long start = t * (long long)(HR * ROWB);
    const long long left = total * (long long)ROWB - start;
    const int nbytes = left <= 0 ? 0 : (int)min(left, (long long)(HR * ROWB));
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(base + (left > 0 ? start : 0)), (short)0, nbytes, 0x00020000);
#pragma unroll
    for (int l = 0; l < LPT; ++l) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (threadIdx.x + HT * l), 0, 0);
      buf[l] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  // the 4 * BD values of batch m: projections 4w .. 4w + 3, dimensions BD m ..
  auto load_batch = [&](double* p, int m) __attribute__((always_inline)) {
    int opaque = 0;
    asm volatile("" : "+s"(opaque));
    const double* pm = proj + opaque + 4 * w * D + BD * m;
#pragma unroll
    for (int t = 0; t < 4 * BD; ++t) p[t] = pm[(t / BD) * D + t % BD];
  };
  // float32 path: the 4 * BD values of batch m, as load_batch
  auto load_batch32 = [&](float* p, int m) __attribute__((always_inline)) {
    int opaque = 0;
    asm volatile("" : "+s"(opaque));
    const float* pm = proj32 + opaque + 4 * w * D + BD * m;
#pragma unroll
    for (int t = 0; t < 4 * BD; ++t) p[t] = pm[(t / BD) * D + t % BD];
  };
  // element e of the 16-byte chunk held in wd
  auto elem = [&](const uint32_t* wd, int e) __attribute__((always_inline)) -> float {
    if constexpr (sizeof(T) == 2)
      return __uint_as_float(e % 2 ? (wd[e / 2] & 0xffff0000u) : (wd[e / 2] << 16));
    else
      return __uint_as_float(wd[e]);
  };

  uint4 buf[LPT];
  long long tile = blockIdx.x;
  load_tile(buf, tile);
  for (; tile < tiles; tile += gridDim.x) {
    const long long t0 = tile * HR;
    const int nrows = (int)min((long long)HR, total - t0);
#pragma unroll
    for (int l = 0; l < LPT; ++l) {
      const int e = threadIdx.x + HT * l;
      *reinterpret_cast<uint4*>(rows + (e / CPR) * STRIDE + 16 * (e % CPR)) = buf[l];
    }
    __syncthreads();
    load_tile(buf, tile + gridDim.x);
    const unsigned char* xr = rows + r * STRIDE;
    uint32_t bits = 0, undecided = 0;
    if constexpr (!CENTRED) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      float nrm = 0.f;
      float pr[2][4 * BD];
      uint32_t wd[4];
      uint4 u = *reinterpret_cast<const uint4*>(xr);
      load_batch32(pr[0], 0);
#pragma unroll
      for (int m = 0; m < NBAT; ++m) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): batch m and the row's chunk m / BPC
        __builtin_amdgcn_sched_barrier(0);
        if (m % BPC == 0) {
          wd[0] = u.x, wd[1] = u.y, wd[2] = u.z, wd[3] = u.w;
          if (m + BPC < NBAT) u = *reinterpret_cast<const uint4*>(xr + 16 * (m / BPC + 1));
        }
        if (m + 1 < NBAT) load_batch32(pr[(m + 1) & 1], m + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < BD; ++d) {
          const float x = elem(wd, (BD * m + d) % EPC);
          nrm = fmaf(x, x, nrm);
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[b] = fmaf(x, pr[m & 1][b * BD + d], acc[b]);
        }
        // all five sums advance batch by batch (otherwise the compiler may
        // run the projections one after the other over the whole row, with
        // every element of the row held in registers)
        asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(nrm));
      }
      const float xn = __builtin_sqrtf(nrm + 0x1p-100f);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float a = __builtin_fabsf(acc[b]);
        if (a > fmaf(coef[4 * w + b], xn, 0x1p-100f) && a <= 3.40282347e38f)
          bits |= (acc[b] > 0.f ? 1u : 0u) << (4 * w + b);
        else
          undecided |= 1u << (4 * w + b);
      }
    } else {
    const long long i = t0 + min(r, nrows - 1);
    const double* mu = mean + (i / N) * D;
    double acc[4] = {0, 0, 0, 0};
    double pr[2][4 * BD];
    double xv[EPC];
    uint4 u = *reinterpret_cast<const uint4*>(xr);
    load_batch(pr[0], 0);
#pragma unroll
    for (int m = 0; m < NBAT; ++m) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): batch m and the row's chunk m / BPC
      __builtin_amdgcn_sched_barrier(0);
      if (m % BPC == 0) {
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          if constexpr (sizeof(T) == 2)
            xv[e] = (double)bf16_to_f32((uint16_t)(wd[e / 2] >> (16 * (e % 2))));
          else
            xv[e] = (double)__uint_as_float(wd[e]);
        }
        if (m + BPC < NBAT) u = *reinterpret_cast<const uint4*>(xr + 16 * (m / BPC + 1));
      }
      if (m + 1 < NBAT) load_batch(pr[(m + 1) & 1], m + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = 0; d < BD; ++d) {
        const int dim = BD * m + d;
        const double xc = xv[dim % EPC] - mu[dim];
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[b] = __dadd_rn(acc[b], __dmul_rn(xc, pr[m & 1][b * BD + d]));
      }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) bits |= (acc[b] > 0.0 ? 1u : 0u) << (4 * w + b);
    }
    part[w][r] = (uint8_t)bits;
    if constexpr (!CENTRED) part_und[w][r] = (uint8_t)undecided;
    __syncthreads();  // the rows are rewritten by the next tile; both halves of each key are in
    if (threadIdx.x < nrows) {
      keys[t0 + threadIdx.x] = (uint8_t)(part[0][threadIdx.x] | part[1][threadIdx.x]);
      if constexpr (!CENTRED)
        undecided_out[t0 + threadIdx.x] = (uint8_t)(part_und[0][threadIdx.x] | part_und[1][threadIdx.x]);
    }
  }
}

// The undecided key bits of the float32 pass.  A workgroup stages the
// float64 projections in LDS, then each wave walks runs of 256 tokens (four
// flag bytes per lane); the tokens with undecided bits are taken eight at a
// time, lane 8j + b forming bit b of the j-th such token as its float64 sum
// in dimension order, one fused multiply-add per term, as the key is
// defined; lane 8j then writes that token's corrected key.
constexpr int FIXUP_BLOCKS = 512;
template <typename T, int D>
__global__ __launch_bounds__(256) void hash_fixup_kernel(const T* __restrict__ q, const double* __restrict__ proj,
                                                         const uint8_t* __restrict__ undecided,
                                                         uint8_t* __restrict__ keys, long long total) {
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte load
  __shared__ double pl[kHashBits * D];
  for (int t = threadIdx.x; t < kHashBits * D; t += blockDim.x) pl[t] = proj[t];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const long long nwaves = (long long)gridDim.x * (blockDim.x >> 6);
  const long long wid = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  for (long long base = wid * 256; base < total; base += nwaves * 256) {
    const long long i0 = base + 4 * lane;
    uint32_t f4 = 0;
    if (i0 + 4 <= total) {
      f4 = *reinterpret_cast<const uint32_t*>(undecided + i0);  // the flags start 256-byte aligned
    } else {
      for (int j = 0; j < 4 && i0 + j < total; ++j) f4 |= (uint32_t)undecided[i0 + j] << (8 * j);
    }
    // tokens (4 per lane) with undecided bits, in order
    uint64_t lanes = __ballot(f4 != 0u);
    uint32_t mine = f4;  // this lane's flags, consumed token by token
    while (lanes) {
      // gather up to eight tokens: slot j of the round is token tok[j]
      long long tok = -1;
      uint32_t fl = 0;
      int filled = 0;
      while (lanes && filled < 8) {
        const int src = __builtin_ctzll(lanes);
        const uint32_t fsrc = (uint32_t)__shfl((int)mine, src);
        const int j = __builtin_ctz(fsrc) / 8;  // first token of that lane with flags
        const uint32_t fj = (fsrc >> (8 * j)) & 0xffu;
        if (lane / 8 == filled) {
          tok = base + 4 * src + j;
          fl = fj;
        }
        if (lane == src) mine &= ~(0xffu << (8 * j));
        const uint32_t rest = fsrc & ~(0xffu << (8 * j));
        if (rest == 0u) lanes &= lanes - 1;
        ++filled;
      }
      const int b = lane & 7;
      bool pos = false;
      if (tok >= 0 && ((fl >> b) & 1u)) {
        const uint4* src = reinterpret_cast<const uint4*>(q + tok * D);
        uint4 row[D / EPC];
#pragma unroll
        for (int c = 0; c < D / EPC; ++c) row[c] = src[c];
        double acc = 0.0;
#pragma unroll
        for (int c = 0; c < D / EPC; ++c) {
          const uint32_t wd[4] = {row[c].x, row[c].y, row[c].z, row[c].w};
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            const float x = sizeof(T) == 2 ? __uint_as_float(e % 2 ? (wd[e / 2] & 0xffff0000u) : (wd[e / 2] << 16))
                                           : __uint_as_float(wd[e]);
            acc = __fma_rn((double)x, pl[b * D + EPC * c + e], acc);
          }
        }
        pos = acc > 0.0;
      }
      const uint32_t set = (uint32_t)(__ballot(pos) >> (lane & ~7)) & 0xffu;
      if (b == 0 && tok >= 0) keys[tok] = (uint8_t)((keys[tok] & ~fl) | (set & fl));
    }
  }
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

__device__ __forceinline__ int wave_incl_scan(int x) {
  // DPP: shifts by 1, 2, 4, 8 within each row of 16 lanes (a lane whose
  // source lies before its row adds 0), then lane 15 of rows 0 and 2 is added
  // to rows 1 and 3, and lane 31 to rows 2 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// ---------------------------------------------------------- stable sort ----
// One workgroup per head.  A 256-bin histogram gives each key's first
// position (an exclusive scan by four waves); tokens are then placed tile by
// tile in token order, SORT_KPT runs of 64 tokens per wave and tile, so that
// a tile's key loads go out together.  Wave w of a tile takes the contiguous
// tokens t0 + 64 (SORT_KPT w + s) + lane, run s after run s - 1: the rank
// among equal keys inside a run comes from ballots over the 8 key bits,
// offset by the wave's running count of that key (cnt[w][key], advanced by
// the run's lowest lane), and across the waves by an ordered prefix over the
// per-wave counts, so the result is the stable order.
constexpr int SORT_NT = 1024;
constexpr int SORT_NW = SORT_NT / 64;
constexpr int SORT_KPT = 8;  // runs of 64 tokens per wave and tile

__global__ __launch_bounds__(SORT_NT) void perm_sort_kernel(const uint8_t* __restrict__ keys,
                                                            int32_t* __restrict__ perm, int N) {
  __shared__ int hist[256];
  __shared__ int base[256];
  __shared__ int cnt[SORT_NW][256];
  __shared__ int wsum[4];
  const int h = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const uint8_t* kh = keys + (size_t)h * N;
  int32_t* ph = perm + (size_t)h * N;

  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  // eight key loads in flight per thread, then their counts: not one round
  // trip per key
  for (int i0 = tid; i0 < N; i0 += SORT_NT * SORT_KPT) {
    int k[SORT_KPT];
#pragma unroll
    for (int j = 0; j < SORT_KPT; ++j) {
      const int i = i0 + j * SORT_NT;
      k[j] = i < N ? kh[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < SORT_KPT; ++j)
      if (k[j] >= 0) atomicAdd(&hist[k[j]], 1);
  }
  __syncthreads();
  int hv = 0, hinc = 0;
  if (tid < 256) {
    hv = hist[tid];
    hinc = wave_incl_scan(hv);
    if (lane == 63) wsum[w] = hinc;
  }
  __syncthreads();
  if (tid < 256) {
    int off = 0;
    for (int ww = 0; ww < w; ++ww) off += wsum[ww];
    base[tid] = off + hinc - hv;
  }
  __syncthreads();

  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  constexpr int TILE = SORT_NT * SORT_KPT;
  for (int t0 = 0; t0 < N; t0 += TILE) {
    for (int e = tid; e < SORT_NW * 256; e += SORT_NT) (&cnt[0][0])[e] = 0;
    int key[SORT_KPT];
#pragma unroll
    for (int r = 0; r < SORT_KPT; ++r) {
      const int i = t0 + 64 * (SORT_KPT * w + r) + lane;
      key[r] = i < N ? kh[i] : -1;
    }
    __syncthreads();
    int rank[SORT_KPT];
#pragma unroll
    for (int r = 0; r < SORT_KPT; ++r) {
      const bool valid = key[r] >= 0;
      unsigned long long same = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const bool bit = (key[r] >> b) & 1;
        const unsigned long long bb = __ballot(valid && bit);
        same &= bit ? bb : ~bb;
      }
      // every lane of a key reads the wave's count before its lowest lane
      // advances it (one wave: the read instruction precedes the write)
      const int before = valid ? cnt[w][key[r]] : 0;
      rank[r] = before + __popcll(same & lt_mask);
      if (valid && (same & lt_mask) == 0ull) cnt[w][key[r]] = before + __popcll(same);
    }
    __syncthreads();
    if (tid < 256) {
      int run = base[tid];
      for (int ww = 0; ww < SORT_NW; ++ww) {
        const int c = cnt[ww][tid];
        cnt[ww][tid] = run;
        run += c;
      }
      base[tid] = run;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < SORT_KPT; ++r)
      if (key[r] >= 0) ph[cnt[w][key[r]] + rank[r]] = t0 + 64 * (SORT_KPT * w + r) + lane;
    __syncthreads();
  }
}

// The token sort over several workgroups per head.  The head's tokens are
// cut into chunks of CSORT_CHUNK; sort_hist_kernel counts each chunk's keys
// (counts[h][key][chunk]); sort_scan_kernel turns the counts in place into
// each (key, chunk)'s first sorted position: the keys in order, and for each
// key the chunks in token order; sort_scatter_kernel places a chunk's tokens
// from those positions with the ranks of perm_sort_kernel's tile, so that
// equal keys keep their token order across and within the chunks.
constexpr int CSORT_NT = 1024;
constexpr int CSORT_KPT = 4;  // runs of 64 tokens per wave: 4096-token chunks
constexpr int CSORT_CHUNK = CSORT_NT * CSORT_KPT;

__global__ __launch_bounds__(CSORT_NT) void sort_hist_kernel(const uint8_t* __restrict__ keys,
                                                             int32_t* __restrict__ counts, int N, int nch) {
  __shared__ int hist[256];
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const uint8_t* kh = keys + (size_t)h * N;
  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  int k[CSORT_KPT];
#pragma unroll
  for (int r = 0; r < CSORT_KPT; ++r) {
    const int i = c * CSORT_CHUNK + r * CSORT_NT + tid;
    k[r] = i < N ? kh[i] : -1;
  }
#pragma unroll
  for (int r = 0; r < CSORT_KPT; ++r)
    if (k[r] >= 0) atomicAdd(&hist[k[r]], 1);
  __syncthreads();
  if (tid < 256) counts[((size_t)h * 256 + tid) * nch + c] = hist[tid];
}

__global__ __launch_bounds__(256) void sort_scan_kernel(int32_t* __restrict__ counts, int nch) {
  __shared__ int wsum[4];
  const int h = blockIdx.x, b = threadIdx.x, w = b >> 6, lane = b & 63;
  int32_t* row = counts + ((size_t)h * 256 + b) * nch;
  int total = 0;
  for (int c = 0; c < nch; ++c) total += row[c];
  const int inc = wave_incl_scan(total);
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int run = inc - total;
  for (int ww = 0; ww < w; ++ww) run += wsum[ww];
  for (int c = 0; c < nch; ++c) {
    const int v = row[c];
    row[c] = run;
    run += v;
  }
}

__global__ __launch_bounds__(CSORT_NT) void sort_scatter_kernel(const uint8_t* __restrict__ keys,
                                                                const int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ perm, int N, int nch) {
  __shared__ int base[256];
  __shared__ int cnt[SORT_NW][256];
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const uint8_t* kh = keys + (size_t)h * N;
  int32_t* ph = perm + (size_t)h * N;
  const int t0 = c * CSORT_CHUNK;
  for (int e = tid; e < SORT_NW * 256; e += CSORT_NT) (&cnt[0][0])[e] = 0;
  if (tid < 256) base[tid] = offsets[((size_t)h * 256 + tid) * nch + c];
  int key[CSORT_KPT];
#pragma unroll
  for (int r = 0; r < CSORT_KPT; ++r) {
    const int i = t0 + 64 * (CSORT_KPT * w + r) + lane;
    key[r] = i < N ? kh[i] : -1;
  }
  __syncthreads();
  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank[CSORT_KPT];
#pragma unroll
  for (int r = 0; r < CSORT_KPT; ++r) {
    const bool valid = key[r] >= 0;
    unsigned long long same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (key[r] >> b) & 1;
      const unsigned long long bb = __ballot(valid && bit);
      same &= bit ? bb : ~bb;
    }
    // every lane of a key reads the wave's count before its lowest lane
    // advances it (one wave: the read instruction precedes the write)
    const int before = valid ? cnt[w][key[r]] : 0;
    rank[r] = before + __popcll(same & lt_mask);
    if (valid && (same & lt_mask) == 0ull) cnt[w][key[r]] = before + __popcll(same);
  }
  __syncthreads();
  if (tid < 256) {
    int run = base[tid];
    for (int ww = 0; ww < SORT_NW; ++ww) {
      const int n = cnt[ww][tid];
      cnt[ww][tid] = run;
      run += n;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < CSORT_KPT; ++r)
    if (key[r] >= 0) ph[cnt[w][key[r]] + rank[r]] = t0 + 64 * (CSORT_KPT * w + r) + lane;
}

// ---------------------------------------------------------------- top-k ----
// One workgroup per (head, group) score row.  Scores are non-negative floats,
// so their bit patterns order like the values, and the k-th largest pattern T
// is found exactly by radix passes over bits [31:21], [20:10], [9:0]; the
// output is every index with score > T and the lowest-index (k - #greater)
// indices with score == T, in ascending index order.
//
// The usual case reads the row once.  A sample of whole 32-key lines (one
// line drawn at a hashed position in each of up to 128 equal strata of the
// row) gives two of its order statistics around the rank k * s / N, wide
// enough that about 0.7 * CAP / 2 keys of the row are expected between them
// (CAP, the LDS capacity in scores, is TK_CAP or, for short rows,
// TK_CAP_SHORT).  The read of the rest of the row then keeps one LDS bit per
// key above the upper one and the (score, index) pairs of the keys between
// the two.  When fewer than k keys lie above the band, at least k above its
// lower end, and the pairs fit, T lies in the band and is found among the
// pairs in LDS; the winners join the bits and the ordered output comes from
// the bits.  The band only decides which keys are looked at again, never
// which are kept, so a row whose band misses T (the sample is a spatially
// clustered one) is still exact: it falls back to the passes below.
//
// The fallback (and the retained-mass variant, whose k comes from its own
// passes) reads the row for the first pass; when T's first-pass bin holds at
// most CAP / 2 scores the second read is also the last (bits for the keys
// above the bin, pairs for the bin); when it holds at most CAP scores they
// are copied to LDS and the ordered output takes a third read; otherwise
// every pass reads the row.  Rows longer than TK_MASK_KEYS keys skip the
// band and the bits.
constexpr int TK_NT = 256;
constexpr int TK_CAP = 4096;
// Rows of at most TK_SHORT_WORDS * 32 keys use TK_CAP_SHORT: 2.25 KB less of
// LDS for the pairs, with the row's bits, keeps a workgroup within a sixth of
// the CU's 160 KB (in 512-byte granules), and the kernel is compiled for six
// waves per SIMD, so six workgroups share a CU instead of five.
constexpr int TK_CAP_SHORT = 3520;
constexpr int TK_SHORT_WORDS = 1074;
constexpr int TK_MASK_KEYS = 1 << 17;  // longest row of the mask path (16 KB of LDS)
constexpr int TK_SAMPLE_LINES = 128;   // 32-key lines of the band's sample (16 keys per thread)


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

// The bin of a radix pass that holds the krem-th largest counted element:
// found[0] = bin, found[1] = elements in higher bins, found[2] = its count.
// Thread t owns bins [t * nb / TK_NT, (t + 1) * nb / TK_NT).
__device__ __forceinline__ void radix_find_bin(int nb, int krem, const int* hist, int* sh, int* found) {
  const int tid = threadIdx.x;
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
}

// The same for two ranks at once: rank rA over histogram hA and rank rB over
// hB (each thread owning `per` bins of each; hB may equal hA).  A rank
// outside [1, count] finds nothing.  found[0..2] for A, found[3..5] for B.
__device__ __forceinline__ void radix_find_bin2(const int* hA, const int* hB, int per, int rA, int rB, int* sh,
                                                int* found) {
  const int tid = threadIdx.x;
  int a = 0, b = 0;
  for (int i = 0; i < per; ++i) {
    a += hA[tid * per + i];
    b += hB[tid * per + i];
  }
  int ea, eb, ta, tb;
  block_excl_scan2(a, b, &ea, &eb, &ta, &tb, sh);
  int above_a = ta - ea - a, above_b = tb - eb - b;
  if (above_a < rA && above_a + a >= rA) {
    for (int i = per - 1; i >= 0; --i) {
      const int bin = tid * per + i;
      if (above_a + hA[bin] >= rA) {
        found[0] = bin;
        found[1] = above_a;
        found[2] = hA[bin];
        break;
      }
      above_a += hA[bin];
    }
  }
  if (above_b < rB && above_b + b >= rB) {
    for (int i = per - 1; i >= 0; --i) {
      const int bin = tid * per + i;
      if (above_b + hB[bin] >= rB) {
        found[3] = bin;
        found[4] = above_b;
        found[5] = hB[bin];
        break;
      }
      above_b += hB[bin];
    }
  }
  __syncthreads();
}

// Line of stratum i of the band's sample: strata split the row's nlines
// 32-key lines into nls runs of equal length (+-1); the line is drawn from
// its run by a multiplicative hash of i.
__device__ __forceinline__ int sample_line(int i, int nls, int nlines) {
  const int a = i * nlines / nls, b = (i + 1) * nlines / nls;
  return a + (int)(((uint32_t)i * 2654435761u) >> 7) % (b - a);
}

// Fixed-point value of a score for the retained-mass budget: floor(x * 2^48)
// for the non-negative float32 with bit pattern x (x = m * 2^(e - 150) with
// the 24-bit significand m of a normal number; zero and subnormals give 0).
__device__ __forceinline__ unsigned long long mass_units(uint32_t x) {
  const int e = (int)(x >> 23);
  if (e == 0) return 0ull;
  const unsigned long long m = (x & 0x7fffffu) | 0x800000u;
  const int sft = e - 102;
  if (sft >= 0) return sft < 40 ? (m << sft) : ~0ull;
  return -sft >= 64 ? 0ull : (m >> -sft);
}

__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long x) {
  const int lane = __lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int src = (lane - off) << 2;
    const uint32_t lo = __builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(x >> 32));
    if (lane >= off) x += ((unsigned long long)hi << 32) | lo;
  }
  return x;
}

// The budget of one group under a retained-mass target: the fewest keys, in
// the top-k order (score descending, index ascending), whose fixed-point
// scores sum to at least ceil(mass * glen * 2^48), at most cap, at least 1.
// Three histogram passes (counts and sums per bin, the same bit fields as the
// top-k) find the score T* at which the running sum from the top reaches the
// target; the keys above T* and just enough of those equal to T* make the
// count.  Reads the row three times.
__device__ __forceinline__ int topk_mass_count(const uint32_t* __restrict__ row, int N, float mass, int glen, int cap,
                                               int* hist, unsigned long long* hsum, unsigned long long* shq, int* sh,
                                               int* found) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NW = TK_NT / 64;
  const unsigned long long target =
      (unsigned long long)ceil((double)mass * (double)glen * 281474976710656.0);  // * 2^48
  unsigned long long rem = target;
  int above = 0;
  uint32_t prefix = 0, pmask = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int b = tid; b < 2048; b += TK_NT) {
      hist[b] = 0;
      hsum[b] = 0ull;
    }
    __syncthreads();
    for (int j0 = 4 * tid; j0 < N; j0 += 4 * TK_NT) {
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
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j0 + e < N && (u[e] & pmask) == prefix) {
          const int b = (u[e] >> shift) & (nb - 1);
          atomicAdd(&hist[b], 1);
          atomicAdd(&hsum[b], mass_units(u[e]));
        }
    }
    __syncthreads();
    // thread t owns bins [t*per, (t+1)*per); sums above a thread = total - inclusive
    const int per = nb / TK_NT;
    unsigned long long msum = 0ull;
    int mcnt = 0;
    for (int b = 0; b < per; ++b) {
      msum += hsum[tid * per + b];
      mcnt += hist[tid * per + b];
    }
    const unsigned long long incl = wave_incl_scan_u64(msum);
    if (lane == 63) shq[w] = incl;
    int ecnt, unused_e, tcnt, unused_t;
    block_excl_scan2(mcnt, 0, &ecnt, &unused_e, &tcnt, &unused_t, sh);  // synchronises shq too
    unsigned long long wbefore = 0ull, total = 0ull;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      if (ww < w) wbefore += shq[ww];
      total += shq[ww];
    }
    if (tid == 0) found[0] = -1;
    __syncthreads();
    unsigned long long asum = total - (wbefore + incl);   // sums of the bins above this thread's
    int acnt = tcnt - ecnt - mcnt;
    if (asum < rem && asum + msum >= rem) {
      for (int b = per - 1; b >= 0; --b) {
        const int bin = tid * per + b;
        if (asum + hsum[bin] >= rem) {
          found[0] = bin;
          found[1] = acnt;
          shq[NW] = asum;
          break;
        }
        asum += hsum[bin];
        acnt += hist[bin];
      }
    }
    __syncthreads();
    if (found[0] < 0) return cap;  // even every key falls short: all are needed
    prefix |= (uint32_t)found[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    above += found[1];
    rem -= shq[NW];
    __syncthreads();
  }
  const unsigned long long unit = mass_units(prefix);
  const long long need = unit ? (long long)((rem + unit - 1) / unit) : 1;
  const long long n = (long long)above + need;
  return (int)(n < 1 ? 1 : (n > cap ? cap : n));
}

// One workgroup per (head, group) row of N scores: the keep[h] / block
// largest (ties to the lower index), written ascending, and their number
// (in keys) to count[h][g].  With block > 1 the row holds scores of whole key
// blocks and every kept block b is written as its keys b*block .. b*block +
// block - 1.  With MASS the number kept is the retained-mass budget of the
// group (capped at keep[h]); groups are runs of G of the nq queries.  Plain
// score rows (keep, idx_start and count null): every row keeps kfix, row g
// writes idx + g * kfix.
template <bool MASS, int CAP, int WAVES>
__global__ __launch_bounds__(TK_NT, WAVES) void group_topk_kernel(const float* __restrict__ colsum, int ldc,
                                                                  int32_t* __restrict__ idx,
                                                                  int32_t* __restrict__ count,
                                                                  const int32_t* __restrict__ keep,
                                                                  const int64_t* __restrict__ idx_start, int head0,
                                                                  int ng, int N, int G, int nq, int block,
                                                                  float keep_mass, int mask_words, int kfix) {
  __shared__ int hist[2048];
  // candidates: CAP scores, or (band and mask paths) up to CAP / 2
  // (score, index) pairs
  __shared__ unsigned long long cand64[CAP / 2];
  uint32_t* cand = reinterpret_cast<uint32_t*>(cand64);
  // one bit per key of the row (dynamic, mask_words words; 0 if the row is
  // too long for the mask path)
  extern __shared__ uint32_t mask[];
  // one bit per 32-key line: lines read by the band's sample
  __shared__ uint32_t sampled[TK_MASK_KEYS / 32 / 32];
  __shared__ unsigned long long hsum[MASS ? 2048 : 1];
  __shared__ unsigned long long shq[TK_NT / 64 + 1];
  __shared__ int sh[8];
  __shared__ int found[6];
  __shared__ int nband;
  const int tid = threadIdx.x;
  const int g = blockIdx.x, hl = blockIdx.y, h = head0 + hl;
  const uint32_t* row = reinterpret_cast<const uint32_t*>(colsum + ((size_t)hl * ng + g) * ldc);
  const int kh = keep ? keep[h] : kfix;
  int k = kh / block;
  int32_t* out = idx + (idx_start ? idx_start[h] : 0) + (int64_t)g * kh;
  if constexpr (MASS) k = topk_mass_count(row, N, keep_mass, min(G, nq - g * G), k, hist, hsum, shq, sh, found);
  if (tid == 0 && count) count[(size_t)h * ng + g] = k * block;

  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  const bool band = !MASS && N <= 32 * mask_words;
  // Reads the row in steps of 16 * TK_NT keys and hands each score to f.
  // Load v of a step covers 4 * TK_NT consecutive keys, four per thread, so
  // each wave reads whole 128-byte lines, and the next step's loads are in
  // flight while this step's scores are handed over.  Keys past the row (and,
  // with skip_sampled, keys of the band's sample lines) are not handed over;
  // their loads read the row's first 16 bytes instead, which stay cached.
  // The row stride is at least N rounded up to 4, so a 16-byte read at any
  // key j < N (j a multiple of 4) stays inside the row.
  // A thread's chunk j = 1024 q + 4 tid lies in line 32 q + tid / 8, so its
  // sample bit is bit tid / 8 of sampled[q]; skipm caches it for q < 64.
  uint64_t skipm = 0;
  // Chunks whose four scores all lie below floor_bits are not handed over.
  auto scan_row = [&](auto f, bool skip_sampled, uint32_t floor_bits) {  // f(score bits, key index)
    constexpr int STEP = 16 * TK_NT;
    auto live = [&](int j) {
      if (!skip_sampled) return j < N;
      const int q = j >> 10;
      const uint32_t smp = q < 64 ? (uint32_t)(skipm >> q) : sampled[q] >> (tid >> 3);
      return j < N && !(smp & 1u);
    };
    auto load = [&](uint4* x, int base) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = base + 4 * (TK_NT * v + tid);
        x[v] = *reinterpret_cast<const uint4*>(row + (live(j) ? j : 0));
      }
    };
    uint4 cur[4], nxt[4];
    load(cur, 0);
    for (int base = 0; base < N; base += STEP) {
      load(nxt, base + STEP);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = base + 4 * (TK_NT * v + tid);
        if (live(j) && max(max(cur[v].x, cur[v].y), max(cur[v].z, cur[v].w)) >= floor_bits) {
          f(cur[v].x, j);
          if (j + 1 < N) f(cur[v].y, j + 1);
          if (j + 2 < N) f(cur[v].z, j + 2);
          if (j + 3 < N) f(cur[v].w, j + 3);
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) cur[v] = nxt[v];
    }
  };
  bool in_lds = false, mask_mode = false;
  int ncand = 0, first_pass = 0;

  if (band) {
    // ---- the band: sample, two of its order statistics, one read of the rest
    const int nlines = (N + 31) >> 5;
    const int nls = min(TK_SAMPLE_LINES, nlines);
    for (int wd = tid; wd < (nlines + 31) >> 5; wd += TK_NT) sampled[wd] = 0u;
    for (int wd = tid; wd < mask_words; wd += TK_NT) mask[wd] = 0u;
    if (tid == 0) nband = 0;
    __syncthreads();
    // 16 sample keys per thread: 16-byte chunk c = tid + TK_NT * v is quarter
    // c & 7 of sample line c >> 3; sv has a bit per slot that holds a key
    uint32_t su[16];
    uint32_t sv = 0u;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = tid + TK_NT * v, i = c >> 3;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (i < nls) {
        const int line = sample_line(i, nls, nlines);
        const int j0 = 32 * line + 4 * (c & 7);
        if (j0 < N) x = *reinterpret_cast<const uint4*>(row + j0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j0 + e < N) sv |= 1u << (4 * v + e);
        if ((c & 7) == 0) atomicOr(&sampled[line >> 5], 1u << (line & 31));
      }
      su[4 * v] = x.x;
      su[4 * v + 1] = x.y;
      su[4 * v + 2] = x.z;
      su[4 * v + 3] = x.w;
    }
    // keys in the sample: only the row's last line can be short
    const int ns = 32 * nls - (sample_line(nls - 1, nls, nlines) == nlines - 1 ? 32 * nlines - N : 0);
    // the expected rank of T in the sample, +- a margin of about
    // 0.35 * CAP / 2 keys of the row.  hi and lo bracket the sample's
    // r_hi-th and r_lo-th largest to 21 bits: a pass over bits [31:21] finds
    // both ranks' bins, a pass over bits [20:11] (one 1024-bin half of the
    // histogram per rank) their sub-bins; hi is the top of its sub-bin, lo
    // the bottom of its own, so the band only grows.
    const float rs = (float)k * (float)ns / (float)N;
    const float dm = 0.35f * (float)(CAP / 2) * (float)ns / (float)N;
    const int r_hi = (int)floorf(rs - dm), r_lo = (int)ceilf(rs + dm);
    const bool has_hi = r_hi >= 1, has_lo = r_lo <= ns;
    for (int b = tid; b < 2048; b += TK_NT) hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if ((sv >> e) & 1u) atomicAdd(&hist[su[e] >> 21], 1);
    __syncthreads();
    radix_find_bin2(hist, hist, 2048 / TK_NT, has_hi ? r_hi : 0, has_lo ? r_lo : 0, sh, found);
    const uint32_t top_hi = (uint32_t)found[0], top_lo = (uint32_t)found[3];
    const int rh = r_hi - found[1], rl = r_lo - found[4];
    __syncthreads();
    for (int b = tid; b < 2048; b += TK_NT) hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if ((sv >> e) & 1u) {
        const int sub = (su[e] >> 11) & 1023;
        if (has_hi && (su[e] >> 21) == top_hi) atomicAdd(&hist[sub], 1);
        if (has_lo && (su[e] >> 21) == top_lo) atomicAdd(&hist[1024 + sub], 1);
      }
    __syncthreads();
    radix_find_bin2(hist, hist + 1024, 1024 / TK_NT, has_hi ? rh : 0, has_lo ? rl : 0, sh, found);
    const uint32_t hi = has_hi ? (top_hi << 21) | ((uint32_t)found[0] << 11) | 0x7ffu : 0xffffffffu;
    const uint32_t lo = has_lo ? (top_lo << 21) | ((uint32_t)found[3] << 11) : 0u;
    __syncthreads();
    int nab = 0;
    auto classify = [&](uint32_t x, int j) {
      if (x > hi) {
        atomicOr(&mask[j >> 5], 1u << (j & 31));
        ++nab;
      } else if (x >= lo) {
        const int slot = atomicAdd(&nband, 1);
        if (slot < CAP / 2) cand64[slot] = ((unsigned long long)x << 32) | (uint32_t)j;
      }
    };
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = tid + TK_NT * v, i = c >> 3;
      if (i < nls) {
        const int j0 = 32 * sample_line(i, nls, nlines) + 4 * (c & 7);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((sv >> (4 * v + e)) & 1u) classify(su[4 * v + e], j0 + e);
      }
    }
    for (int q = 0; q < min(64, (N + 1023) >> 10); ++q)
      skipm |= (uint64_t)((sampled[q] >> (tid >> 3)) & 1u) << q;
    scan_row(classify, true, lo);
    int unused_e0, unused_e1, above, unused_t;
    block_excl_scan2(nab, 0, &unused_e0, &unused_e1, &above, &unused_t, sh);  // also orders nband and the LDS
    const int nb_keys = nband;
    if (above < k && above + nb_keys >= k && nb_keys <= CAP / 2) {
      // T lies in the band: the remaining passes run over its pairs, from
      // the first pass whose bits lo and hi do not share (pairs lie in
      // [lo, hi], so they share those bits too)
      ncand = nb_keys;
      krem = k - above;
      in_lds = mask_mode = true;
      if ((lo >> 21) == (hi >> 21)) {
        first_pass = 1;
        prefix = lo & (0x7ffu << 21);
        pmask = 0x7ffu << 21;
        if ((lo >> 10) == (hi >> 10)) {
          first_pass = 2;
          prefix = lo & ~0x3ffu;
          pmask = ~0x3ffu;
        }
      }
    }
    __syncthreads();
  }

  for (int pass = first_pass; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int b = tid; b < 2048; b += TK_NT) hist[b] = 0;
    __syncthreads();
    auto count = [&](uint32_t x, int) {
      if ((x & pmask) == prefix) atomicAdd(&hist[(x >> shift) & (nb - 1)], 1);
    };
    if (in_lds) {
      for (int c = tid; c < ncand; c += TK_NT)
        count(mask_mode ? (uint32_t)(cand64[c] >> 32) : cand[c], 0);
    } else {
      scan_row(count, false, prefix);
    }
    __syncthreads();
    radix_find_bin(nb, krem, hist, sh, found);
    prefix |= (uint32_t)found[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    krem -= found[1];
    const int in_bin = found[2];
    __syncthreads();
    if (!in_lds && pass == 0 && in_bin <= CAP / 2 && N <= 32 * mask_words) {
      // second (and last) read of the row: the keys above T's bin are kept,
      // one bit each; the (score, index) pairs of the bin go to LDS
      for (int wd = tid; wd < mask_words; wd += TK_NT) mask[wd] = 0u;
      if (tid == 0) sh[0] = 0;
      __syncthreads();
      scan_row([&](uint32_t x, int j) {
        if ((x & pmask) > prefix)
          atomicOr(&mask[j >> 5], 1u << (j & 31));
        else if ((x & pmask) == prefix)
          cand64[atomicAdd(&sh[0], 1)] = ((unsigned long long)x << 32) | (uint32_t)j;
      }, false, prefix);
      __syncthreads();
      ncand = in_bin;
      in_lds = mask_mode = true;
    } else if (!in_lds && pass == 0 && in_bin <= CAP) {
      // second read: the scores in T's bin, to LDS (exactly in_bin of them)
      if (tid == 0) sh[0] = 0;
      __syncthreads();
      scan_row([&](uint32_t x, int) {
        if ((x & pmask) == prefix) cand[atomicAdd(&sh[0], 1)] = x;
      }, false, prefix);
      __syncthreads();
      ncand = in_bin;
      in_lds = true;
    }
  }
  const uint32_t T = prefix;

  if (mask_mode) {
    // the pairs' winners join the mask: scores above T, and of the scores
    // equal to T the krem with the lowest indices
    int neq = 0;
    for (int c = tid; c < ncand; c += TK_NT) {
      const unsigned long long e = cand64[c];
      const uint32_t x = (uint32_t)(e >> 32);
      if (x > T) atomicOr(&mask[(uint32_t)e >> 5], 1u << ((uint32_t)e & 31));
      neq += x == T;
    }
    int neq_e0, neq_e1, neq_all, neq_t1;
    block_excl_scan2(neq, 0, &neq_e0, &neq_e1, &neq_all, &neq_t1, sh);
    // ties: the krem-th smallest index J among the pairs equal to T, as the
    // krem-th largest of ~j (radix passes over the pairs); krem == neq_all
    // (the usual single key at T) keeps them all
    uint32_t jkey = 0;
    if (krem < neq_all) {
      uint32_t pre = 0, pm = 0;
      int r = krem;
      for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nb = pass == 2 ? 1024 : 2048;
        for (int b = tid; b < 2048; b += TK_NT) hist[b] = 0;
        __syncthreads();
        for (int c = tid; c < ncand; c += TK_NT) {
          const unsigned long long e = cand64[c];
          const uint32_t nj = ~(uint32_t)e;
          if ((uint32_t)(e >> 32) == T && (nj & pm) == pre) atomicAdd(&hist[(nj >> shift) & (nb - 1)], 1);
        }
        __syncthreads();
        radix_find_bin(nb, r, hist, sh, found);
        pre |= (uint32_t)found[0] << shift;
        pm |= (uint32_t)(nb - 1) << shift;
        r -= found[1];
        __syncthreads();
      }
      jkey = pre;
    }
    for (int c = tid; c < ncand; c += TK_NT) {
      const unsigned long long e = cand64[c];
      if ((uint32_t)(e >> 32) == T && ~(uint32_t)e >= jkey)
        atomicOr(&mask[(uint32_t)e >> 5], 1u << ((uint32_t)e & 31));
    }
    __syncthreads();
    // ordered compaction of the mask into an LDS window of CAP positions
    // (the pairs' space, free now), which then goes out with consecutive
    // stores; one window per CAP kept keys.  Words are taken in rounds of
    // TK_NT, one per thread, so a run of full words spreads over the lanes.
    const int nwords = (N + 31) / 32;
    int32_t* stage = reinterpret_cast<int32_t*>(cand64);
    for (int w0 = 0; w0 < k; w0 += CAP) {
      const int wn = min(CAP, k - w0);
      int base = 0;  // kept keys in the rounds before
      for (int r0 = 0; r0 < nwords && base < w0 + wn; r0 += TK_NT) {
        const int wd = r0 + tid;
        const uint32_t word = wd < nwords ? mask[wd] : 0u;
        const int cnt = __popc(word);
        int ex, unused_e, tot, unused_t;
        block_excl_scan2(cnt, 0, &ex, &unused_e, &tot, &unused_t, sh);
        int pos = base + ex;
        if (pos < w0 + wn && pos + cnt > w0) {
          uint32_t bits = word;
          while (bits) {
            const int j = 32 * wd + __ffs(bits) - 1;
            bits &= bits - 1;
            if (pos >= w0 && pos < w0 + wn) stage[pos - w0] = j;
            ++pos;
          }
        }
        base += tot;
      }
      __syncthreads();
      if (block == 1) {
        for (int e = tid; e < wn; e += TK_NT) out[w0 + e] = stage[e];
      } else {
        for (int e = tid; e < wn * block; e += TK_NT) out[(int64_t)w0 * block + e] = stage[e / block] * block + e % block;
      }
      __syncthreads();
    }
    return;
  }

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

// V rounded to float16 (nearest even) for the selection's P·V products, one
// head per blockIdx.y, eight values per thread and step, scaled by 2^-e
// (e = 0 in the first pass).  The first pass also records the head's
// largest magnitude as a bit pattern (non-negative floats order like
// unsigned integers; infinities and NaNs lie above every finite value).
__device__ __forceinline__ uint4 v_f16_chunk(uint4 x, int e, uint32_t* amax) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    *amax = max(*amax, max((w[k] << 16) & 0x7fffffffu, w[k] & 0x7fff0000u));
    const float a = __builtin_ldexpf(__uint_as_float(w[k] << 16), -e);
    const float b = __builtin_ldexpf(__uint_as_float(w[k] & 0xffff0000u), -e);
    const f16x2 hv = {(_Float16)a, (_Float16)b};
    o[k] = __builtin_bit_cast(uint32_t, hv);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__global__ __launch_bounds__(256) void v_to_f16_kernel(const uint4* __restrict__ v, uint4* __restrict__ out,
                                                       long long per8, uint32_t* __restrict__ hmax) {
  const size_t base = (size_t)blockIdx.y * per8;
  uint32_t amax = 0;
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  // four 16-byte loads in flight per thread, then their conversions
  for (; i + 3 * stride < per8; i += 4 * stride) {
    uint4 a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = v[base + i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) out[base + i + u * stride] = v_f16_chunk(a[u], 0, &amax);
  }
  for (; i < per8; i += stride) out[base + i] = v_f16_chunk(v[base + i], 0, &amax);
  // one atomic per workgroup: the wave maxima meet in LDS first
  __shared__ uint32_t wmax[4];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(&hmax[blockIdx.y], max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
}

// The second pass: e = the smallest power of two that brings the head's
// largest finite magnitude below 65520 (where float16 rounding overflows),
// 0 when it is already below or V is not finite; heads with e > 0 are
// rounded again.  vexp[head] = e for the attention kernels' epilogues.
__global__ __launch_bounds__(256) void v_f16_rescale_kernel(const uint4* __restrict__ v, uint4* __restrict__ out,
                                                            long long per8, const uint32_t* __restrict__ hmax,
                                                            int* __restrict__ vexp) {
  const uint32_t m = hmax[blockIdx.y];
  int e = 0;
  if (m >= 0x477ff000u && m < 0x7f800000u) {  // 65520 <= max < infinity
    const float mx = __uint_as_float(m);
    while (__builtin_ldexpf(mx, -e) >= 65520.f) ++e;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) vexp[blockIdx.y] = e;
  if (e == 0) return;
  const size_t base = (size_t)blockIdx.y * per8;
  uint32_t unused = 0;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < per8; i += (long long)gridDim.x * blockDim.x)
    out[base + i] = v_f16_chunk(v[base + i], e, &unused);
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
  if (tok >= T * Y * X) {  // past the grid: the trailing tokens keep their order
    for (int h = 0; h < H; ++h) perm[(size_t)h * N + tok] = tok;
    return;
  }
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

// count[h][g] = keep[h]: every group keeps its head's full budget.
__global__ void fill_counts_kernel(int32_t* __restrict__ count, const int32_t* __restrict__ keep, long long total,
                                   int ng) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long long)gridDim.x * blockDim.x)
    count[i] = keep[i / ng];
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
void hash_launch(const void* q, const double* proj, const double* mean, uint8_t* keys, uint8_t* undecided,
                 long long total, int N, hipStream_t s) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const long long tiles = (total + HR - 1) / HR;
  const dim3 grid((unsigned)std::min<long long>(tiles, (long long)std::max(cus, 1) * HASH_BLOCKS_PER_CU));
  const float* proj32 = reinterpret_cast<const float*>(proj + kHashBits * D);
  const float* coef = proj32 + kHashBits * D;
  if (mean) {
    hipLaunchKernelGGL((hash_keys_kernel<T, D, true>), grid, dim3(HT), 0, s, static_cast<const T*>(q), proj, proj32,
                       coef, mean, keys, undecided, total, N);
  } else {
    hipLaunchKernelGGL((hash_keys_kernel<T, D, false>), grid, dim3(HT), 0, s, static_cast<const T*>(q), proj,
                       proj32, coef, mean, keys, undecided, total, N);
    const long long fblocks = std::min<long long>(FIXUP_BLOCKS, (total + 1023) / 1024);
    hipLaunchKernelGGL((hash_fixup_kernel<T, D>), dim3((unsigned)fblocks), dim3(256), 0, s, static_cast<const T*>(q),
                       proj, undecided, keys, total);
  }
}
// Sort key of each group's launch order: floor(m * 256 / N) for its median
// kept key m (entry count/2 of the ascending list), one thread per group.
__global__ __launch_bounds__(256) void group_bucket_kernel(const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ count,
                                                           const int32_t* __restrict__ keep,
                                                           const int64_t* __restrict__ idx_start,
                                                           uint8_t* __restrict__ bucket, int head0, int nheads, int ng,
                                                           int N, long long total_idx) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long long)nheads * ng) return;
  const int h = head0 + (int)(t / ng), g = (int)(t % ng);
  long long start;
  int n;
  group_keys(keep, idx_start, count, h, g, N, ng, total_idx, &start, &n);
  const int m = clamp_index(idx[start + n / 2], N);
  bucket[(size_t)h * ng + g] = (uint8_t)(((long long)m * 256) / N);
}

}  // namespace

hipError_t launch_hash_keys(const void* q, int dtype, const double* proj, const double* mean, uint8_t* keys,
                            uint8_t* undecided, int H, int N, int D, hipStream_t s) {
  const long long total = (long long)H * N;
  if (total == 0) return hipSuccess;
  if (dtype == 1) {
    if (D == 64)
      hash_launch<uint16_t, 64>(q, proj, mean, keys, undecided, total, N, s);
    else
      hash_launch<uint16_t, 128>(q, proj, mean, keys, undecided, total, N, s);
  } else {
    if (D == 64)
      hash_launch<float, 64>(q, proj, mean, keys, undecided, total, N, s);
    else
      hash_launch<float, 128>(q, proj, mean, keys, undecided, total, N, s);
  }
  return launched(s);
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
  return launched(s);
}

hipError_t launch_v_to_f16(const void* v, void* out, int nheads, long long per_head, uint32_t* hmax, int* vexp,
                           hipStream_t s) {
  if (nheads == 0 || per_head == 0) return hipSuccess;
  if (per_head % 8) return hipErrorInvalidValue;
  hipError_t e = launch_zero_floats(reinterpret_cast<float*>(hmax), nheads, s);
  if (e != hipSuccess) return e;
  const long long per8 = per_head / 8;
  // about 4096 workgroups over all heads, a few 16-byte chunks per thread
  const long long bx = std::max<long long>(1, std::min<long long>((per8 + 255) / 256, (4096 + nheads - 1) / nheads));
  const dim3 grid((unsigned)bx, (unsigned)nheads);
  hipLaunchKernelGGL(v_to_f16_kernel, grid, dim3(256), 0, s, static_cast<const uint4*>(v), static_cast<uint4*>(out),
                     per8, hmax);
  if ((e = launched(s)) != hipSuccess) return e;
  hipLaunchKernelGGL(v_f16_rescale_kernel, grid, dim3(256), 0, s, static_cast<const uint4*>(v),
                     static_cast<uint4*>(out), per8, static_cast<const uint32_t*>(hmax), vexp);
  return launched(s);
}

int sort_chunks(int N) { return (N + CSORT_CHUNK - 1) / CSORT_CHUNK; }

hipError_t launch_perm_sort(const uint8_t* keys, int32_t* perm, int32_t* counts, int H, int N, hipStream_t s) {
  if (H == 0 || N == 0) return hipSuccess;
  const int nch = sort_chunks(N);
  hipLaunchKernelGGL(sort_hist_kernel, dim3((unsigned)nch, (unsigned)H), dim3(CSORT_NT), 0, s, keys, counts, N, nch);
  hipError_t e = launched(s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sort_scan_kernel, dim3((unsigned)H), dim3(256), 0, s, counts, nch);
  if ((e = launched(s)) != hipSuccess) return e;
  hipLaunchKernelGGL(sort_scatter_kernel, dim3((unsigned)nch, (unsigned)H), dim3(CSORT_NT), 0, s, keys, counts, perm,
                     N, nch);
  return launched(s);
}

hipError_t launch_group_topk(const float* colsum, int ldc, int32_t* idx, int32_t* count, const int32_t* keep,
                             const int64_t* idx_start, int head0, int nheads, int ng, int N, int G, int nq, int block,
                             float keep_mass, hipStream_t s) {
  if (nheads == 0 || ng == 0) return hipSuccess;
  // the kernel's 16-byte reads at keys j < N need a row stride of at least N
  // rounded up to 4 keys, and 16-byte aligned rows
  if (ldc % 4 != 0 || ldc < N) return hipErrorInvalidValue;
  // the band and mask paths of the top-k hold one bit per key in LDS (rows
  // up to TK_MASK_KEYS keys); longer rows take the three-read path
  const int mask_words = N <= TK_MASK_KEYS ? (N + 31) / 32 : 0;
  const size_t lds = (size_t)mask_words * 4;
  if (keep_mass > 0.f)
    hipLaunchKernelGGL((group_topk_kernel<true, TK_CAP, 1>), dim3(ng, nheads), dim3(TK_NT), lds, s, colsum, ldc, idx,
                       count, keep, idx_start, head0, ng, N, G, nq, block, keep_mass, mask_words, 0);
  else if (mask_words <= TK_SHORT_WORDS)
    hipLaunchKernelGGL((group_topk_kernel<false, TK_CAP_SHORT, 6>), dim3(ng, nheads), dim3(TK_NT), lds, s, colsum, ldc,
                       idx, count, keep, idx_start, head0, ng, N, G, nq, block, keep_mass, mask_words, 0);
  else
    hipLaunchKernelGGL((group_topk_kernel<false, TK_CAP, 1>), dim3(ng, nheads), dim3(TK_NT), lds, s, colsum, ldc, idx,
                       count, keep, idx_start, head0, ng, N, G, nq, block, keep_mass, mask_words, 0);
  return launched(s);
}

hipError_t launch_topk_rows(const float* scores, int ld, int rows, int n, int k, int32_t* idx, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (ld % 4 != 0 || ld < n || k < 1 || k > n) return hipErrorInvalidValue;
  const int mask_words = n <= TK_MASK_KEYS ? (n + 31) / 32 : 0;
  if (mask_words <= TK_SHORT_WORDS)
    hipLaunchKernelGGL((group_topk_kernel<false, TK_CAP_SHORT, 6>), dim3(rows, 1), dim3(TK_NT), (size_t)mask_words * 4,
                       s, scores, ld, idx, nullptr, nullptr, nullptr, 0, rows, n, 1, n, 1, 0.f, mask_words, k);
  else
    hipLaunchKernelGGL((group_topk_kernel<false, TK_CAP, 1>), dim3(rows, 1), dim3(TK_NT), (size_t)mask_words * 4, s,
                       scores, ld, idx, nullptr, nullptr, nullptr, 0, rows, n, 1, n, 1, 0.f, mask_words, k);
  return launched(s);
}

hipError_t launch_group_order(const int32_t* idx, const int32_t* count, const int32_t* keep,
                              const int64_t* idx_start, uint8_t* bucket, int32_t* order, int head0, int nheads, int ng,
                              int N, long long total_idx, hipStream_t s) {
  const long long total = (long long)nheads * ng;
  if (total == 0 || N == 0) return hipSuccess;
  hipLaunchKernelGGL(group_bucket_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, idx, count, keep,
                     idx_start, bucket, head0, nheads, ng, N, total_idx);
  const hipError_t e = launched(s);
  if (e != hipSuccess) return e;
  // the stable counting sort of the grouping, over ng keys per head
  hipLaunchKernelGGL(perm_sort_kernel, dim3(nheads), dim3(SORT_NT), 0, s, bucket + (size_t)head0 * ng,
                     order + (size_t)head0 * ng, ng);
  return launched(s);
}

hipError_t launch_fill_counts(int32_t* count, const int32_t* keep, int H, int ng, hipStream_t s) {
  const long long total = (long long)H * ng;
  if (total == 0) return hipSuccess;
  const long long blocks = std::min<long long>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(fill_counts_kernel, dim3((unsigned)blocks), dim3(256), 0, s, count, keep, total, ng);
  return launched(s);
}

hipError_t launch_block_scores(const float* colsum, int ldc, float* bs, int ldb, long long rows, int nb,
                               hipStream_t s) {
  const long long total = rows * nb;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(block_scores_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, colsum, ldc, bs,
                     ldb, rows, nb);
  return launched(s);
}

hipError_t launch_iota_perm(int32_t* perm, int H, int N, hipStream_t s) {
  const long long total = (long long)H * N;
  if (total == 0) return hipSuccess;
  const long long blocks = std::min<long long>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(iota_perm_kernel, dim3((unsigned)blocks), dim3(256), 0, s, perm, total, N);
  return launched(s);
}

hipError_t launch_morton_perm(int32_t* perm, int H, int N, int T, int Y, int X, hipStream_t s) {
  if (H == 0 || N == 0) return hipSuccess;
  hipLaunchKernelGGL(morton_perm_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, perm, H, N, T, Y, X);
  return launched(s);
}

hipError_t launch_zero_floats(float* p, long long n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const long long blocks = std::min<long long>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(zero_floats_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return launched(s);
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
    const hipError_t e = launched(s);
    if (e != hipSuccess) return e;
    done += chunk;
  }
  return hipSuccess;
}

}  // namespace mcs
