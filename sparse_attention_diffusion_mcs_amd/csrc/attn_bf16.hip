// bf16 attention kernels for gfx950 (MFMA v_mfma_f32_16x16x32_bf16, float32
// accumulation): dense attention with the per-group key scores of the
// selection step, and gathered-KV sparse attention of the reuse step.
//
// Method: abstract of "MC-Sparse: Deconstructing and Closing the Dense-Sparse
// Attention Gap in Diffusion Transformers" (exact probabilities drive the
// choice of individual KV tokens per tile-aligned query group; the residual
// between dense and sparse outputs is cached and reused), and section "What
// Trips People Up" of "The quality cliff nobody admits to" (the sparse
// softmax is renormalised over the kept tokens; the residual corrects it).
//
// Work decomposition.  One workgroup owns a tile of query rows: 32 rows per
// wave (two 16-row MFMA blocks).  For the sparse modes the tile is exactly one
// query group (G = 64 -> 2 waves, G = 128 -> 4 waves), so every wave shares
// the group's gathered KV tile.  The loop walks KV tiles of 64 tokens: the
// workgroup gathers K rows (row-major, padded) and V rows (transposed, two
// tokens packed per 32-bit word) into LDS; each wave computes S^T = K Q^T so
// that every lane ends up holding scores of a single query row; the online
// softmax then needs one in-lane pass plus two cross-lane steps, and the
// probabilities are already laid out as the B operand of O^T += V^T P^T.
#include "device.h"
#include "launch.h"

namespace mcs {
namespace {

constexpr int BKV = 64;  // KV tokens per tile

// Position of token t (0..63) of a KV tile inside a transposed V row.  The S^T
// accumulator gives lane-quad q the tokens {16h + 4q + i} of each 32-token
// chunk (h = 0, 1; i = 0..3); this order makes those 8 tokens contiguous so
// that the V^T operand of the PV product is a single 16-byte LDS read.
__device__ __forceinline__ int vpos(int t) {
  return (t & ~31) | ((t & 12) << 1) | ((t & 16) >> 2) | (t & 3);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

template <int D, int NW, int MODE>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int KK = D / 32;          // 32-wide k-steps of QK^T
  constexpr int DB = D / 16;          // 16-wide output column blocks
  constexpr int KS = D + 8;           // K tile row stride (elements), 16 B pad
  constexpr int VS = BKV + 8;         // V^T tile row stride (elements), 16 B pad
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int UK = BKV * CH / NT;   // K chunks per thread per tile
  constexpr int UV = (BKV / 2) * CH / NT;  // V token-pair chunks per thread per tile
  constexpr bool SPARSE = (MODE == MODE_REUSE || MODE == MODE_RESINIT);
  static_assert(UK * NT == BKV * CH && UV * NT == (BKV / 2) * CH, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) __bf16 ks[BKV * KS];
  __shared__ __attribute__((aligned(16))) __bf16 vt[D * VS];
  __shared__ float red[MODE == MODE_SELECT ? NW : 1][BKV];
  __shared__ float lse_s[MODE == MODE_SELECT ? BM : 1];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
  const int N = a.N;

  // ---- work item -------------------------------------------------------
  const int tiles = SPARSE ? a.ng : (N + BM - 1) / BM;
  const int L = xcd_remap(blockIdx.x, a.nheads * tiles, a.run);
  const int hs = L / tiles, tile = L % tiles;
  const int h = (MODE == MODE_REUSE) ? clamp_index(a.sched[hs], a.H) : a.head0 + hs;
  const int row0 = tile * BM;
  const size_t hoff = (size_t)h * N * D;
  const uint16_t* qh = static_cast<const uint16_t*>(a.q) + hoff;
  const uint16_t* kh = static_cast<const uint16_t*>(a.k) + hoff;
  const uint16_t* vh = static_cast<const uint16_t*>(a.v) + hoff;
  const int32_t* permh = a.perm ? a.perm + (size_t)h * N : nullptr;

  int nkv = N;
  const int32_t* kvidx = nullptr;
  if constexpr (SPARSE) {
    long long start;
    group_keys(a.keep, a.idx_start, h, tile, N, a.total_idx, &start, &nkv);
    kvidx = a.idx + start;
  }
  const int nt = (nkv + BKV - 1) / BKV;
  const float sl2 = a.scale * kLog2e;

  // ---- Q fragments: lane holds row (16 rb + lr) of its wave, dims 8 lq + 32 kk ..
  bf16x8 qf[2][KK];
  int rtok[2];
  bool rvalid[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int p = row0 + 32 * w + 16 * rb + lr;
    rvalid[rb] = p < N;
    rtok[rb] = (MODE == MODE_PLAIN) ? p : (rvalid[rb] ? clamp_index(permh[p], N) : 0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (rvalid[rb]) u = *reinterpret_cast<const uint4*>(qh + (size_t)rtok[rb] * D + 8 * lq + 32 * kk);
      qf[rb][kk] = as_bf16x8(u);
    }
  }

  // ---- KV tile staging --------------------------------------------------
  uint4 kreg[UK];
  uint4 vreg[UV][2];
  auto gload = [&](int j) {
#pragma unroll
    for (int i = 0; i < UK; ++i) {
      const int u = tid + NT * i, t = u / CH, c = u % CH, tk = j * BKV + t;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (tk < nkv) {
        const int row = SPARSE ? clamp_index(kvidx[tk], N) : tk;
        x = *reinterpret_cast<const uint4*>(kh + (size_t)row * D + 8 * c);
      }
      kreg[i] = x;
    }
#pragma unroll
    for (int i = 0; i < UV; ++i) {
      const int u = tid + NT * i, pp = u % (BKV / 2), c = u / (BKV / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int tk = j * BKV + 2 * pp + e;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (tk < nkv) {
          const int row = SPARSE ? clamp_index(kvidx[tk], N) : tk;
          x = *reinterpret_cast<const uint4*>(vh + (size_t)row * D + 8 * c);
        }
        vreg[i][e] = x;
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < UK; ++i) {
      const int u = tid + NT * i, t = u / CH, c = u % CH;
      *reinterpret_cast<uint4*>(ks + t * KS + 8 * c) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < UV; ++i) {
      const int u = tid + NT * i, pp = u % (BKV / 2), c = u / (BKV / 2);
      const int pos = vpos(2 * pp);
      const uint32_t* x0 = reinterpret_cast<const uint32_t*>(&vreg[i][0]);
      const uint32_t* x1 = reinterpret_cast<const uint32_t*>(&vreg[i][1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = __builtin_amdgcn_perm(x1[e], x0[e], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(x1[e], x0[e], 0x07060302u);
        *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * e) * VS + pos) = lo;
        *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * e + 1) * VS + pos) = hi;
      }
    }
  };

  // ---- pass 1: online-softmax attention over the KV tiles ---------------
  float m_run[2] = {-1e30f, -1e30f};
  float l_run[2] = {0.f, 0.f};
  f32x4 oacc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) oacc[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore();
  __syncthreads();
  for (int j = 0; j < nt; ++j) {
    if (j + 1 < nt) gload(j + 1);

    // S^T[token][row]: lane holds tokens 16 tb + 4 lq + i of row 16 rb + lr
    f32x4 s[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) s[tb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + (16 * tb + lr) * KS + 8 * lq + 32 * kk);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          s[tb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rb][kk], s[tb][rb], 0, 0, 0);
      }
    }
    const int vcols = nkv - j * BKV;
    if (vcols < BKV) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * tb + 4 * lq + i >= vcols) {
            s[tb][0][i] = -INFINITY;
            s[tb][1][i] = -INFINITY;
          }
    }

    bf16x8 pf[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float mx = s[0][rb][0];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[tb][rb][i]);
      mx = fmaxf(mx, xor_shfl(mx, 16));
      mx = fmaxf(mx, xor_shfl(mx, 32));
      const float mnew = fmaxf(m_run[rb], mx * sl2);
      const float alpha = fast_exp2(m_run[rb] - mnew);
      m_run[rb] = mnew;
      float ls = 0.f;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(fmaf(s[tb][rb][i], sl2, -mnew));
          s[tb][rb][i] = p;
          ls += p;
        }
      l_run[rb] = l_run[rb] * alpha + ls;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db][rb] *= alpha;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        bf16x8 t;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          t[i] = (__bf16)s[2 * kc][rb][i];
          t[4 + i] = (__bf16)s[2 * kc + 1][rb][i];
        }
        pf[kc][rb] = t;
      }
    }

    // O^T[dim][row] += V^T P^T
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vt + (16 * db + lr) * VS + 32 * kc + 8 * lq);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          oacc[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[kc][rb], oacc[db][rb], 0, 0, 0);
      }
    }
    __syncthreads();
    if (j + 1 < nt) lstore();
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    float l = l_run[rb];
    l += xor_shfl(l, 16);
    l += xor_shfl(l, 32);
    const float inv = 1.0f / l;
    const int r = 32 * w + 16 * rb + lr;
    const int p = row0 + r;
    if constexpr (MODE == MODE_SELECT) {
      if (lq == 0) lse_s[r] = rvalid[rb] ? m_run[rb] + __log2f(l) : INFINITY;
    }
    if (!rvalid[rb]) continue;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 16 * db + 4 * lq;
      const f32x4 o = oacc[db][rb] * inv;
      if constexpr (MODE == MODE_PLAIN) {
        uint16_t* out = static_cast<uint16_t*>(a.o) + hoff + (size_t)p * D + col;
        *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      } else if constexpr (MODE == MODE_SELECT) {
        *reinterpret_cast<f32x4*>(a.residual + hoff + (size_t)p * D + col) = o;
        if (a.o) {
          uint16_t* out = static_cast<uint16_t*>(a.o) + hoff + (size_t)rtok[rb] * D + col;
          *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        }
      } else if constexpr (MODE == MODE_REUSE) {
        const f32x4 res = *reinterpret_cast<const f32x4*>(a.residual + hoff + (size_t)p * D + col);
        const f32x4 y = o + res;
        uint16_t* out = static_cast<uint16_t*>(a.o) + hoff + (size_t)rtok[rb] * D + col;
        *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
      } else {  // MODE_RESINIT
        f32x4* rp = reinterpret_cast<f32x4*>(a.residual + hoff + (size_t)p * D + col);
        *rp = *rp - o;
      }
    }
  }
  if constexpr (MODE != MODE_SELECT) return;

  // ---- pass 2 (selection): per-group key scores c(j) = sum_i exp(s_ij - lse_i)
  __syncthreads();
  float nlse[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) nlse[rb][i] = -lse_s[32 * w + 16 * rb + 4 * lq + i];

  constexpr int WPG_MAX = 4;  // waves per group (G / 32)
  const int wpg = a.G / 32;
  const int gpt = BM / a.G;   // groups per tile
  (void)WPG_MAX;
  gload(0);
  lstore();
  __syncthreads();
  for (int j = 0; j < nt; ++j) {
    if (j + 1 < nt) gload(j + 1);
    // S[row][token]: lane holds rows 16 rb + 4 lq + i of token 16 tb + lr
    f32x4 s[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) s[rb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + (16 * tb + lr) * KS + 8 * lq + 32 * kk);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          s[rb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[rb][kk], kf, s[rb][tb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      float cs = 0.f;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) cs += fast_exp2(fmaf(s[rb][tb][i], sl2, nlse[rb][i]));
      cs += xor_shfl(cs, 16);
      cs += xor_shfl(cs, 32);
      if (lq == 0) red[w][16 * tb + lr] = cs;
    }
    __syncthreads();
    for (int t = tid; t < gpt * BKV; t += NT) {
      const int gi = t / BKV, col = t % BKV, tok = j * BKV + col;
      const int g = row0 / a.G + gi;
      if (tok < N && g < a.ng) {
        float sum = 0.f;
        for (int ww = 0; ww < wpg; ++ww) sum += red[gi * wpg + ww][col];
        a.colsum[((size_t)hs * a.ng + g) * a.ldc + tok] = sum;
      }
    }
    if (j + 1 < nt) lstore();
    __syncthreads();
  }
}

template <int D, int NW, int MODE>
hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  constexpr int BM = NW * 32;
  const int tiles = (MODE == MODE_REUSE || MODE == MODE_RESINIT) ? a.ng : (a.N + BM - 1) / BM;
  const long long nblocks = (long long)a.nheads * tiles;
  if (nblocks == 0) return hipSuccess;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_bf16_kernel<D, NW, MODE>), dim3((unsigned)nblocks), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int mode, const AttnArgs& a, hipStream_t s) {
  switch (mode) {
    case MODE_PLAIN: return launch_one<D, 4, MODE_PLAIN>(a, s);
    case MODE_SELECT: return launch_one<D, 4, MODE_SELECT>(a, s);
    case MODE_REUSE:
      return a.G == 64 ? launch_one<D, 2, MODE_REUSE>(a, s) : launch_one<D, 4, MODE_REUSE>(a, s);
    case MODE_RESINIT:
      return a.G == 64 ? launch_one<D, 2, MODE_RESINIT>(a, s) : launch_one<D, 4, MODE_RESINIT>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_bf16(int mode, const AttnArgs& a, hipStream_t s) {
  if (a.D == 64) return launch_d<64>(mode, a, s);
  if (a.D == 128) return launch_d<128>(mode, a, s);
  return hipErrorInvalidValue;
}

}  // namespace mcs
