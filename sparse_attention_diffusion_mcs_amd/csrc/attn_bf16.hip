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
// Work decomposition.  A workgroup owns a tile of query rows, 32 rows per wave
// (two 16-row MFMA blocks).  In the sparse modes the tile is exactly one query
// group (G = 64 -> 2 waves, G = 128 -> 4 waves), so all waves share the
// group's gathered KV tiles; in the dense modes it is 128 rows (4 waves).
//
// KV tiles of 32 tokens are gathered straight from global memory into LDS
// with global_load_lds_dwordx4 (no staging registers), double-buffered with
// one barrier per tile.  Rows are stored with an XOR swizzle of their 16-byte
// chunks chosen so that both LDS read patterns are free of bank conflicts: the
// K operand (16-byte reads, 16 rows per quarter-wave) and the V operand, read
// transposed with ds_read_b64_tr_b16 (8 rows x 2 chunks per half-wave).
//
// Each wave computes S^T = K Q^T, so every lane holds scores of one query row;
// the row max needs one in-lane pass and two cross-lane steps, and the
// probabilities are already in the B-operand layout of O^T += V^T P^T.  The
// running max is only moved (and O, l rescaled) when a row's tile max exceeds
// it by more than 2^8; otherwise probabilities up to 2^8 are accumulated
// against the stale max, which leaves O / l unchanged.
#include "device.h"
#include "launch.h"

namespace mcs {
namespace {

constexpr int BKV = 32;             // KV tokens per tile
constexpr float kRescaleSlack = 8.0f;  // log2 units

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int D>
struct Geo {
  static constexpr int ROWB = D * 2;           // bytes per K/V row
  static constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;         // rows per wave-wide 1 KB load
  static constexpr int NI = BKV / RPI;         // 1 KB loads per tensor per tile
  static constexpr int TILE = BKV * ROWB;      // bytes per tensor per tile
  // Stored position of 16-byte chunk c of tile row t is c ^ swz(t).
  __device__ static __forceinline__ int swz(int t) {
    if constexpr (D == 128)
      return ((t & 7) << 1) | ((t >> 3) & 1);
    else
      return (((t >> 1) & 3) << 1) | ((t >> 3) & 1);
  }
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D, int NW, int MODE>
__global__ __launch_bounds__(NW * 64, 2) void attn_bf16_kernel(AttnArgs a) {
  using GE = Geo<D>;
  constexpr int BM = NW * 32;
  constexpr int KK = D / 32;                 // k-steps of QK^T
  constexpr int DB = D / 16;                 // output column blocks
  constexpr int UPW = GE::NI / NW;           // loads per tensor per tile per wave
  constexpr bool SPARSE = (MODE == MODE_REUSE || MODE == MODE_RESINIT);
  constexpr int STAGE = 2 * GE::TILE;        // K tile + V tile
  static_assert(UPW * NW == GE::NI, "tile loads must split evenly over the waves");

  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];
  __shared__ float red[MODE == MODE_SELECT ? 2 : 1][NW][BKV];
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

  // ---- tile loads -------------------------------------------------------
  // Load u of this wave covers tile rows ii*RPI .. +RPI-1 (ii = w + NW u); lane
  // `lane` fills stored chunk (lane % CPR) of row ii*RPI + lane / CPR.
  auto tile_row_of = [&](int u) { return (w + NW * u) * GE::RPI + lane / GE::CPR; };
  auto source_row = [&](int j, int u) -> int {
    const int tk = j * BKV + tile_row_of(u);
    if constexpr (SPARSE) {
      return clamp_index(kvidx[tk < nkv ? tk : nkv - 1], N);
    } else {
      return tk < N ? tk : N - 1;
    }
  };
  int rows_next[UPW];
  auto issue = [&](int j, int stage, bool with_v) {
    char* kt = lds + stage * STAGE;
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
      const int t = tile_row_of(u);
      const int c = (lane % GE::CPR) ^ GE::swz(t);
      const size_t off = (size_t)rows_next[u] * D + 8 * c;
      const int ii = w + NW * u;
      __builtin_amdgcn_global_load_lds(kh + off, (lds_void*)(kt + ii * 1024), 16, 0, 0);
      if (with_v) __builtin_amdgcn_global_load_lds(vh + off, (lds_void*)(kt + GE::TILE + ii * 1024), 16, 0, 0);
    }
    (void)j;
  };
  auto fetch_rows = [&](int j) {
    if (j < nt) {
#pragma unroll
      for (int u = 0; u < UPW; ++u) rows_next[u] = source_row(j, u);
    }
  };

  // K operand (A of S^T, or B of S): tile row 16 tb + lr, chunk lq + 4 kk
  auto kfrag = [&](const char* kt, int tb, int kk) -> bf16x8 {
    const int t = 16 * tb + lr;
    const int c = (lq + 4 * kk) ^ GE::swz(t);
    return *reinterpret_cast<const bf16x8*>(kt + t * GE::ROWB + 16 * c);
  };
  // V^T operand for output column block db: two transposed 8-byte reads of
  // tokens 4 lq + lr/4 (+16), dims 16 db + 4 (lr % 4) ..
  auto vfrag = [&](const char* vt, int db) -> bf16x8 {
    uint2 x[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int t = 16 * hh + 4 * lq + (lr >> 2);
      const int c = (2 * db + ((lr & 3) >> 1)) ^ GE::swz(t);
      const char* p = vt + t * GE::ROWB + 16 * c + 8 * (lr & 1);
      x[hh] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p));
    }
    return as_bf16x8(make_uint4(x[0].x, x[0].y, x[1].x, x[1].y));
  };

  // ---- pass 1: online-softmax attention over the KV tiles ---------------
  float m_run[2] = {-1e30f, -1e30f};
  float l_run[2] = {0.f, 0.f};
  f32x4 oacc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) oacc[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  fetch_rows(0);
  issue(0, 0, true);
  fetch_rows(1);
  for (int j = 0; j < nt; ++j) {
    wait_vm();
    __syncthreads();
    if (j + 1 < nt) {
      issue(j + 1, (j + 1) & 1, true);
      fetch_rows(j + 2);
    }
    const char* kt = lds + (j & 1) * STAGE;
    const char* vt = kt + GE::TILE;

    // S^T[token][row]: lane holds tokens 16 tb + 4 lq + i of row 16 rb + lr
    f32x4 s[2][2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) s[tb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const bf16x8 kf = kfrag(kt, tb, kk);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          s[tb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rb][kk], s[tb][rb], 0, 0, 0);
      }
    }
    const int vcols = nkv - j * BKV;
    if (vcols < BKV) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * tb + 4 * lq + i >= vcols) {
            s[tb][0][i] = -INFINITY;
            s[tb][1][i] = -INFINITY;
          }
    }

    float mx[2];
    bool need = false;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float m = fmaxf(fmaxf(s[0][rb][0], s[0][rb][1]), fmaxf(s[0][rb][2], s[0][rb][3]));
      m = fmaxf(m, fmaxf(fmaxf(s[1][rb][0], s[1][rb][1]), fmaxf(s[1][rb][2], s[1][rb][3])));
      m = fmaxf(m, xor_shfl(m, 16));
      m = fmaxf(m, xor_shfl(m, 32));
      mx[rb] = m * sl2;
      need |= mx[rb] > m_run[rb] + kRescaleSlack;
    }
    if (__ballot(need) != 0ull) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float mnew = fmaxf(m_run[rb], mx[rb]);
        const float alpha = fast_exp2(m_run[rb] - mnew);
        m_run[rb] = mnew;
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db][rb] *= alpha;
      }
    }
    bf16x8 pf[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float ls = 0.f;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(fmaf(s[tb][rb][i], sl2, -m_run[rb]));
          s[tb][rb][i] = p;
          ls += p;
        }
      l_run[rb] += ls;
      pf[rb] = as_bf16x8(make_uint4(pack_bf16x2(s[0][rb][0], s[0][rb][1]), pack_bf16x2(s[0][rb][2], s[0][rb][3]),
                                    pack_bf16x2(s[1][rb][0], s[1][rb][1]), pack_bf16x2(s[1][rb][2], s[1][rb][3])));
    }

    // O^T[dim][row] += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 vf = vfrag(vt, db);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        oacc[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rb], oacc[db][rb], 0, 0, 0);
    }
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

  const int wpg = a.G / 32;   // waves per group
  const int gpt = BM / a.G;   // groups per tile
  auto flush = [&](int j) {   // cross-wave sums of tile j -> colsum
    for (int t = tid; t < gpt * BKV; t += NW * 64) {
      const int gi = t / BKV, col = t % BKV, tok = j * BKV + col;
      const int g = row0 / a.G + gi;
      if (tok < N && g < a.ng) {
        float sum = 0.f;
        for (int ww = 0; ww < wpg; ++ww) sum += red[j & 1][gi * wpg + ww][col];
        a.colsum[((size_t)hs * a.ng + g) * a.ldc + tok] = sum;
      }
    }
  };
  fetch_rows(0);
  issue(0, 0, false);
  fetch_rows(1);
  for (int j = 0; j < nt; ++j) {
    wait_vm();
    __syncthreads();
    if (j + 1 < nt) {
      issue(j + 1, (j + 1) & 1, false);
      fetch_rows(j + 2);
    }
    if (j > 0) flush(j - 1);
    const char* kt = lds + (j & 1) * STAGE;
    // S[row][token]: lane holds rows 16 rb + 4 lq + i of token 16 tb + lr
    f32x4 s[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) s[rb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const bf16x8 kf = kfrag(kt, tb, kk);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          s[rb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[rb][kk], kf, s[rb][tb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      float cs = 0.f;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) cs += fast_exp2(fmaf(s[rb][tb][i], sl2, nlse[rb][i]));
      cs += xor_shfl(cs, 16);
      cs += xor_shfl(cs, 32);
      if (lq == 0) red[j & 1][w][16 * tb + lr] = cs;
    }
  }
  __syncthreads();
  if (nt > 0) flush(nt - 1);
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
