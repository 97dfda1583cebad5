// float32 attention kernels (plain VALU arithmetic), the float32 counterpart of
// attn_bf16.hip for small float32 problems: dense attention (with the
// per-group key scores of the selection step) and gathered-KV sparse
// attention of the reuse step.  Same method references as attn_bf16.hip.
//
// One thread owns one query row; a workgroup owns one query tile (one query
// group in the group-ordered modes).  KV tiles of 32 tokens are staged in LDS
// and read by all threads as broadcasts.
#include "device.h"
#include "launch.h"

namespace mcs {
namespace {

constexpr int BKVF = 32;

template <int D, int MODE>
__global__ __launch_bounds__(128) void attn_f32_kernel(AttnArgs a) {
  constexpr bool SPARSE = (MODE == MODE_REUSE || MODE == MODE_RESINIT);
  __shared__ float ksh[BKVF][D];
  __shared__ float vsh[BKVF][D];
  __shared__ float red[MODE == MODE_SELECT ? 128 : 1][BKVF + 1];

  const int BM = blockDim.x;
  const int tid = threadIdx.x;
  const int N = a.N;
  const int tiles = (MODE == MODE_PLAIN) ? (N + BM - 1) / BM : a.ng;
  const int L = xcd_remap(blockIdx.x, a.nheads * tiles, a.run);
  const int hs = L / tiles, wt = L % tiles;
  const int h = (MODE == MODE_REUSE) ? clamp_index(a.sched[hs], a.H) : a.head0 + hs;
  // the sparse passes take a head's groups in the metadata's launch order
  const int tile = (SPARSE && a.order) ? clamp_index(a.order[(size_t)h * a.ng + wt], a.ng) : wt;
  const size_t hoff = (size_t)h * N * D;
  const float* qh = static_cast<const float*>(a.q) + hoff;
  const float* kh = static_cast<const float*>(a.k) + hoff;
  const float* vh = static_cast<const float*>(a.v) + hoff;

  const int p = tile * BM + tid;
  const bool valid = p < N;
  const int tok = (MODE == MODE_PLAIN) ? p : (valid ? clamp_index(a.perm[(size_t)h * N + p], N) : 0);

  int nkv = N;
  const int32_t* kvidx = nullptr;
  if constexpr (SPARSE) {
    long long start;
    group_keys(a.keep, a.idx_start, a.count, h, tile, N, a.ng, a.total_idx, &start, &nkv);
    kvidx = a.idx + start;
  }

  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = valid ? qh[(size_t)tok * D + c] : 0.f;
    o[c] = 0.f;
  }
  float m = -1e30f, l = 0.f;

  auto load_tile = [&](int j0, int cnt) {
    for (int e = tid; e < BKVF * D; e += BM) {
      const int t = e / D, c = e % D;
      float kx = 0.f, vx = 0.f;
      if (t < cnt) {
        const int row = SPARSE ? clamp_index(kvidx[j0 + t], N) : j0 + t;
        kx = kh[(size_t)row * D + c];
        vx = vh[(size_t)row * D + c];
      }
      ksh[t][c] = kx;
      vsh[t][c] = vx;
    }
  };

  for (int j0 = 0; j0 < nkv; j0 += BKVF) {
    const int cnt = min(BKVF, nkv - j0);
    load_tile(j0, cnt);
    __syncthreads();
    float sv[BKVF];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < BKVF; ++t) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) s = fmaf(q[c], ksh[t][c], s);
      s *= a.scale;
      sv[t] = (t < cnt) ? s : -INFINITY;
      mx = fmaxf(mx, sv[t]);
    }
    const float mnew = fmaxf(m, mx);
    const float alpha = expf(m - mnew);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] *= alpha;
#pragma unroll
    for (int t = 0; t < BKVF; ++t) {
      const float pr = expf(sv[t] - mnew);
      l += pr;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(pr, vsh[t][c], o[c]);
    }
    m = mnew;
    __syncthreads();
  }

  const float inv = 1.0f / l;
  if (valid) {
    // float32 problems keep a float32 residual
    float* resrow = a.residual ? static_cast<float*>(a.residual) + hoff + (size_t)p * D : nullptr;
    if constexpr (MODE == MODE_PLAIN) {
      float* out = static_cast<float*>(a.o) + hoff + (size_t)p * D;
#pragma unroll
      for (int c = 0; c < D; ++c) out[c] = o[c] * inv;
    } else if constexpr (MODE == MODE_SELECT) {
#pragma unroll
      for (int c = 0; c < D; ++c) resrow[c] = o[c] * inv;
      if (a.o) {
        float* out = static_cast<float*>(a.o) + hoff + (size_t)tok * D;
#pragma unroll
        for (int c = 0; c < D; ++c) out[c] = o[c] * inv;
      }
    } else if constexpr (MODE == MODE_REUSE) {
      float* out = static_cast<float*>(a.o) + hoff + (size_t)tok * D;
#pragma unroll
      for (int c = 0; c < D; ++c) out[c] = o[c] * inv + resrow[c];
    } else {
#pragma unroll
      for (int c = 0; c < D; ++c) resrow[c] = resrow[c] - o[c] * inv;
    }
  }
  if constexpr (MODE != MODE_SELECT) return;

  // pass 2: group key scores c(j) = sum over the group's rows of exp(s_ij - lse_i)
  const float lse = valid ? m + logf(l) : INFINITY;
  for (int j0 = 0; j0 < N; j0 += BKVF) {
    const int cnt = min(BKVF, N - j0);
    load_tile(j0, cnt);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < BKVF; ++t) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) s = fmaf(q[c], ksh[t][c], s);
      red[tid][t] = expf(s * a.scale - lse);
    }
    __syncthreads();
    if (tid < cnt) {
      float sum = 0.f;
      for (int r = 0; r < BM; ++r) sum += red[r][tid];
      a.colsum[((size_t)hs * a.ng + tile) * a.ldc + j0 + tid] = sum;
    }
    __syncthreads();
  }
}

template <int D, int MODE>
hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  const int bm = (MODE == MODE_PLAIN) ? 64 : a.G;
  const int tiles = (MODE == MODE_PLAIN) ? (a.N + bm - 1) / bm : a.ng;
  const long long nblocks = (long long)a.nheads * tiles;
  if (nblocks == 0) return hipSuccess;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_f32_kernel<D, MODE>), dim3((unsigned)nblocks), dim3(bm), 0, s, a);
  return launched(s);
}

template <int D>
hipError_t launch_d(int mode, const AttnArgs& a, hipStream_t s) {
  switch (mode) {
    case MODE_PLAIN: return launch_one<D, MODE_PLAIN>(a, s);
    case MODE_SELECT: return launch_one<D, MODE_SELECT>(a, s);
    case MODE_REUSE: return launch_one<D, MODE_REUSE>(a, s);
    case MODE_RESINIT: return launch_one<D, MODE_RESINIT>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_f32(int mode, const AttnArgs& a, hipStream_t s) {
  if (a.D == 64) return launch_d<64>(mode, a, s);
  if (a.D == 128) return launch_d<128>(mode, a, s);
  return hipErrorInvalidValue;
}

}  // namespace mcs
