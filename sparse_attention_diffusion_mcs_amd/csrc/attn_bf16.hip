// bf16 attention kernels for gfx950 (MFMA v_mfma_f32_16x16x32_bf16, float32
// accumulation; the selection passes take their P·V products on
// v_mfma_f32_16x16x32_f16): dense attention with the per-group key scores of
// the selection step, and gathered-KV sparse attention of the reuse step.
//
// Method: abstract of "MC-Sparse: Deconstructing and Closing the Dense-Sparse
// Attention Gap in Diffusion Transformers" (exact probabilities drive the
// choice of individual KV tokens per tile-aligned query group; the residual
// between dense and sparse outputs is cached and reused), and section "What
// Trips People Up" of "The quality cliff nobody admits to" (the sparse
// softmax is renormalised over the kept tokens; the residual corrects it).
//
// Work decomposition.  A workgroup owns a tile of query rows, 32 rows per wave
// (two 16-row MFMA blocks; 64 rows in the key-score pass).  In the sparse modes the tile is exactly one query
// group (G = 64 -> 2 waves, G = 128 -> 4 waves), so all waves share the
// group's gathered KV tiles; in the dense modes it is 128 rows (4 waves).
//
// KV tiles of BK tokens are gathered straight from global memory into LDS with
// buffer_load_dwordx4 ... lds (no staging registers, 32-bit row offsets into
// the head's K and V) into two LDS stages, one barrier per tile.  The two
// stages are distinct LDS objects and the tile loop is unrolled by two, so the
// compiler can see that a tile's reads never alias the copy into the other
// stage and does not wait for that copy before reading.  Rows are stored with
// an XOR swizzle of their 16-byte chunks.  The V operand, read transposed
// with ds_read_b64_tr_b16 (8 rows x 2 chunks per half-wave), is free of bank
// conflicts; the K operand's 16-byte reads, which the LDS serves 32 lanes at
// a time, meet a 2-way conflict (a swizzle free of both costs more address
// registers than the conflict costs time).  All operand reads of a tile are
// issued before its first MFMA so that their latency overlaps.
//
// Each wave computes S^T = K Q^T, so every lane holds scores of one query row
// (a quarter of the tile's tokens; the row's other tokens sit in three lanes
// at distance 16) and the probabilities are already in the B-operand layout
// of O^T += V^T P^T.  The running max is only moved (and O, l rescaled) when
// a row's tile max exceeds it by more than 2^8; otherwise probabilities up to
// 2^8 are accumulated against the stale max, which leaves O / l unchanged.
// The check needs only each lane's own maximum; the row max (two row-swap
// permutes) is formed on the rare rescale.
//
// The selection runs two launches over the same query tiles: the dense pass
// (MODE_SELECT: dense output and each row's log-sum-exp) and the key-score
// pass (MODE_SCORE), which recomputes QK^T and sums each group's exact
// probabilities per key.
#include "device.h"
#include "launch.h"

namespace mcs {
namespace {

constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr int kBufferConfig = 0x00020000;  // raw buffer resource word 3 (gfx9 family)
constexpr long long kScoreItems = 12288;   // key-score work items to aim for (~16 rounds of resident workgroups)

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int D, int BK>
struct Geo {
  static constexpr int ROWB = D * 2;           // bytes per K/V row
  static constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;         // rows per wave-wide 1 KB load
  static constexpr int NI = BK / RPI;          // 1 KB loads per tensor per tile
  static constexpr int TILE = BK * ROWB;       // bytes per tensor per tile
  // Stored position of 16-byte chunk c of tile row t is c ^ swz(t).
  __device__ static __forceinline__ int swz(int t) {
    if constexpr (D == 128)
      return ((t & 7) << 1) | ((t >> 3) & 1);
    else
      return (((t >> 1) & 3) << 1) | ((t >> 3) & 1);
  }
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f16x8 as_f16x8(uint4 u) { return __builtin_bit_cast(f16x8, u); }
// two float32 values rounded to float16 (nearest even), packed
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2 t = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, t);
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D, int NW, int MODE, int BK>
__global__ __launch_bounds__(NW * 64, 2) void attn_bf16_kernel(AttnArgs a) {
  using GE = Geo<D, BK>;
  // Query rows per wave: two 16-row MFMA blocks, or four in the key-score
  // pass, whose registers hold only QK^T operands and scores.
  constexpr int RB = (MODE == MODE_SCORE) ? 4 : 2;
  constexpr int RPW = 16 * RB;
  constexpr int BM = NW * RPW;
  constexpr int KK = D / 32;                 // k-steps of QK^T
  constexpr int DB = D / 16;                 // output column blocks
  constexpr int TB = BK / 16;                // 16-token blocks per tile
  constexpr int KC = BK / 32;                // 32-token chunks of the PV product
  constexpr int UPW = GE::NI / NW;           // loads per tensor per tile per wave
  constexpr bool SPARSE = (MODE == MODE_REUSE || MODE == MODE_RESINIT);
  // The selection step's outputs (dense output and selection-time sparse
  // output) feed the cached residual, which every reuse step adds back; they
  // carry the probabilities into the PV product at more than bf16's 8 bits:
  // the product runs on float16 MFMAs with P in float16 (11 bits) and V from
  // a.v16, V rounded to float16 once per selection after a per-head scaling
  // by 2^-a.v16_exp[head] (0 unless the head's V exceeds float16's range),
  // which the epilogue undoes.
  constexpr bool PRECISE_PV = (MODE == MODE_SELECT || MODE == MODE_RESINIT);
  constexpr int STAGE = 2 * GE::TILE;        // K tile + V tile
  static_assert(UPW * NW == GE::NI, "tile loads must split evenly over the waves");

  __shared__ __attribute__((aligned(1024))) char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[STAGE];
  __shared__ float red[MODE == MODE_SCORE ? 2 : 1][NW][MODE == MODE_SCORE ? 2 * BK : 1];

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = a.N;

  // ---- work item -------------------------------------------------------
  const int tiles = SPARSE ? a.ng : (N + BM - 1) / BM;
  // The key-score pass also splits the keys into kchunks ranges (scores of
  // different keys are independent); its work items run row tile fastest, so
  // the items in flight on an XCD share a key range of one head.
  const int kchunks = (MODE == MODE_SCORE && a.kchunks > 1) ? a.kchunks : 1;
  const int L = xcd_remap(blockIdx.x, a.nheads * tiles * kchunks, a.run);
  const int hs = L / (tiles * kchunks), wt = L % tiles, kc = (L / tiles) % kchunks;
  const int h = (MODE == MODE_REUSE) ? clamp_index(a.sched[hs], a.H) : a.head0 + hs;
  // the sparse passes take a head's groups in the metadata's launch order
  const int tile = (SPARSE && a.order) ? clamp_index(a.order[(size_t)h * a.ng + wt], a.ng) : wt;
  const int row0 = tile * BM;
  const size_t hoff = (size_t)h * N * D;
  const uint16_t* qh = static_cast<const uint16_t*>(a.q) + hoff;
  const uint16_t* kh = static_cast<const uint16_t*>(a.k) + hoff;
  // the float16 copy of V holds the launch's heads only
  const uint16_t* vh = PRECISE_PV ? static_cast<const uint16_t*>(a.v16) + (size_t)(h - a.head0) * N * D
                                  : static_cast<const uint16_t*>(a.v) + hoff;
  const int32_t* permh = a.perm ? a.perm + (size_t)h * N : nullptr;
  // Buffer resources over this head's K and V (N rows of ROWB bytes).
  const int head_bytes = N * GE::ROWB;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)kh, (short)0, head_bytes, kBufferConfig);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)vh, (short)0, head_bytes, kBufferConfig);

  int nkv = N;
  __amdgpu_buffer_rsrc_t ridx;  // the group's kept keys; reads past the end return 0 (row 0)
  if constexpr (SPARSE) {
    long long start;
    group_keys(a.keep, a.idx_start, a.count, h, tile, N, a.ng, a.total_idx, &start, &nkv);
    ridx = __builtin_amdgcn_make_buffer_rsrc((void*)(a.idx + start), (short)0, nkv * 4, kBufferConfig);
  }
  const int nt = (nkv + BK - 1) / BK;
  const float sl2 = a.scale * kLog2e;

  // ---- Q fragments: lane holds row (16 rb + lr) of its wave, dims 8 lq + 32 kk ..
  bf16x8 qf[RB][KK];
  int rtok[RB];
  bool rvalid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int p = row0 + RPW * w + 16 * rb + lr;
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
  // `lane` fills stored chunk (lane % CPR) of row ii*RPI + lane / CPR.  Rows
  // past the end of the key list load key 0 (their scores are masked): the
  // whole index offset goes in the range-checked vector offset, so those
  // index reads return 0.
  // The source row of each load is fetched one tile ahead and only turned into
  // a byte offset when the copy is issued, so that nothing waits on the fetch
  // (and, through the in-order memory counter, on the copy issued before it).
  int src_row[UPW];
  int chunk_off[UPW];
#pragma unroll
  for (int u = 0; u < UPW; ++u) {
    const int t = (w + NW * u) * GE::RPI + lane / GE::CPR;
    chunk_off[u] = 16 * ((lane % GE::CPR) ^ GE::swz(t));
  }
  auto fetch_rows = [&](int j) {
    if (j < nt) {
#pragma unroll
      for (int u = 0; u < UPW; ++u) {
        const int t = (w + NW * u) * GE::RPI + lane / GE::CPR;
        if constexpr (SPARSE)
          src_row[u] = __builtin_amdgcn_raw_buffer_load_b32(ridx, 4 * (BK * j + t), 0, 0);
        else
          src_row[u] = j * BK + t;
      }
    }
  };
  auto issue = [&](char* stage, bool with_v) {
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
      const int ii = w + NW * u;
      // Kept keys come from the metadata, whose indices are < N; an index
      // outside [0, N) in edited metadata makes an offset past the head's
      // buffer range, which the bounds check turns into zeros.  The dense
      // modes clamp the rows of their ragged last tile to the last key.
      const unsigned row = SPARSE ? (unsigned)src_row[u] : min((unsigned)src_row[u], (unsigned)(N - 1));
      const int off = (int)((row * GE::ROWB) | (unsigned)chunk_off[u]);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(stage + ii * 1024), 16, off, 0, 0, 0);
      if (with_v)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(stage + GE::TILE + ii * 1024), 16, off, 0, 0, 0);
    }
  };

  // K operand (A of S^T, or B of S): tile row 16 tb + lr, chunk lq + 4 kk
  auto kfrag = [&](const char* kt, int tb, int kk) -> bf16x8 {
    const int t = 16 * tb + lr;
    const int c = (lq + 4 * kk) ^ GE::swz(t);
    return *reinterpret_cast<const bf16x8*>(kt + t * GE::ROWB + 16 * c);
  };
  // Half of the V^T operand of 32-token chunk kc for output column block db:
  // a transposed 8-byte read of token 32 kc + 16 hh + 4 lq + lr/4, dims
  // 16 db + 4 (lr % 4) ..
  auto vhalf = [&](const char* vt, int kc, int db, int hh) -> uint2 {
    const int t = 32 * kc + 16 * hh + 4 * lq + (lr >> 2);
    const int c = (2 * db + ((lr & 3) >> 1)) ^ GE::swz(t);
    const char* p = vt + t * GE::ROWB + 16 * c + 8 * (lr & 1);
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p));
  };

  if constexpr (MODE != MODE_SCORE) {  // every mode but the key-score pass
    // ---- pass 1: online-softmax attention over the KV tiles ---------------
    float m_run[2] = {-1e30f, -1e30f};
    float l_run[2] = {0.f, 0.f};
    f32x4 oacc[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) oacc[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto attend_tile = [&](int j, const char* cur, char* nxt, auto masked) {
      constexpr bool F16 = PRECISE_PV;  // P and V as float16
      wait_vm<0>();
      __syncthreads();
      if (j + 1 < nt) {
        issue(nxt, true);
        fetch_rows(j + 2);
      }
      const char* vt = cur + GE::TILE;
      bf16x8 kf[KK][TB];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) kf[kk][tb] = kfrag(cur, tb, kk);
      uint2 vr[KC][DB][2];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) vr[kc][db][hh] = vhalf(vt, kc, db, hh);

      // S^T[token][row]: lane holds tokens 16 tb + 4 lq + i of row 16 rb + lr
      f32x4 s[TB][2];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) s[tb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            s[tb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk][tb], qf[rb][kk], s[tb][rb], 0, 0, 0);
      if constexpr (decltype(masked)::value) {  // the ragged last tile only
        const int vcols = nkv - j * BK;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * tb + 4 * lq + i >= vcols) {
              s[tb][0][i] = -INFINITY;
              s[tb][1][i] = -INFINITY;
            }
      }

      // This lane's maximum over its tokens of the tile (log2 units).  Whether
      // some row of the wave needs a rescale, or carries large probabilities,
      // is the same question asked of every lane, so the row maxima across the
      // four lanes of a row are only formed when a rescale happens.
      float lmx[2];
      bool need = false;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float m = s[0][rb][0];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = __builtin_fmaxf(m, s[tb][rb][i]);
        lmx[rb] = m * sl2;
        need |= lmx[rb] > m_run[rb] + kRescaleSlack;
      }
      if (__ballot(need) != 0ull) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const float mnew = __builtin_fmaxf(m_run[rb], quad_rows_max(lmx[rb]));
          const float alpha = fast_exp2(m_run[rb] - mnew);
          m_run[rb] = mnew;
          l_run[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db][rb] *= alpha;
        }
      }
      bf16x8 pf[F16 ? 1 : KC][2];
      f16x8 ph[F16 ? KC : 1][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float ls = 0.f;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(fmaf(s[tb][rb][i], sl2, -m_run[rb]));
            s[tb][rb][i] = p;
            ls = (tb == 0 && i == 0) ? p : ls + p;  // starts at the first term, not 0 + it
          }
        l_run[rb] += ls;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          if constexpr (F16) {
            ph[kc][rb] = as_f16x8(make_uint4(pack_f16x2(s[2 * kc][rb][0], s[2 * kc][rb][1]),
                                             pack_f16x2(s[2 * kc][rb][2], s[2 * kc][rb][3]),
                                             pack_f16x2(s[2 * kc + 1][rb][0], s[2 * kc + 1][rb][1]),
                                             pack_f16x2(s[2 * kc + 1][rb][2], s[2 * kc + 1][rb][3])));
            continue;
          }
          const uint4 hi = make_uint4(pack_bf16x2(s[2 * kc][rb][0], s[2 * kc][rb][1]),
                                      pack_bf16x2(s[2 * kc][rb][2], s[2 * kc][rb][3]),
                                      pack_bf16x2(s[2 * kc + 1][rb][0], s[2 * kc + 1][rb][1]),
                                      pack_bf16x2(s[2 * kc + 1][rb][2], s[2 * kc + 1][rb][3]));
          pf[kc][rb] = as_bf16x8(hi);
        }
      }

      // O^T[dim][row] += V^T P^T
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint4 vu = make_uint4(vr[kc][db][0].x, vr[kc][db][0].y, vr[kc][db][1].x, vr[kc][db][1].y);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            if constexpr (F16)
              oacc[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(vu), ph[kc][rb], oacc[db][rb], 0, 0, 0);
            else
              oacc[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vu), pf[kc][rb], oacc[db][rb], 0, 0, 0);
          }
        }
    };

    fetch_rows(0);
    if (nt > 0) issue(st0, true);
    fetch_rows(1);
    {
      const Flag<false> full;
      const Flag<true> ragged;
      const int nfull = (nkv % BK) ? nt - 1 : nt;   // tiles that need no masking
      int j = 0;
      for (; j + 1 < nfull; j += 2) {
        attend_tile(j, st0, st1, full);
        attend_tile(j + 1, st1, st0, full);
      }
      if (j < nfull) attend_tile(j++, st0, st1, full);
      if (j < nt) {
        if (j & 1)
          attend_tile(j, st1, st0, ragged);
        else
          attend_tile(j, st0, st1, ragged);
      }
    }

    // ---- epilogue ---------------------------------------------------------
    // the float16 V of the selection passes was scaled by 2^-vexp
    const int vexp = PRECISE_PV ? a.v16_exp[h - a.head0] : 0;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float l = quad_rows_sum(l_run[rb]);
      const float inv = PRECISE_PV ? __builtin_ldexpf(1.0f / l, vexp) : 1.0f / l;
      const int r = RPW * w + 16 * rb + lr;
      const int p = row0 + r;
      if constexpr (MODE == MODE_SELECT) {
        if (lq == 0 && rvalid[rb]) a.lse[(size_t)hs * N + p] = m_run[rb] + __log2f(l);
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
          // the float32 dense output goes to the residual region, or (bf16
          // residual) to the workspace until the sparse pass forms the residual
          float* od = a.odense ? a.odense + (size_t)hs * N * D : static_cast<float*>(a.residual) + hoff;
          *reinterpret_cast<f32x4*>(od + (size_t)p * D + col) = o;
          if (a.o) {
            uint16_t* out = static_cast<uint16_t*>(a.o) + hoff + (size_t)rtok[rb] * D + col;
            *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
          }
        } else if constexpr (MODE == MODE_REUSE) {
          f32x4 res;
          if (a.residual_bf16) {
            const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.residual) + hoff +
                                                            (size_t)p * D + col);
            res = f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u), __uint_as_float(r.y << 16),
                        __uint_as_float(r.y & 0xffff0000u)};
          } else {
            res = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.residual) + hoff + (size_t)p * D + col);
          }
          const f32x4 y = o + res;
          uint16_t* out = static_cast<uint16_t*>(a.o) + hoff + (size_t)rtok[rb] * D + col;
          *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
        } else {  // MODE_RESINIT
          if (a.residual_bf16) {
            const f32x4 od = *reinterpret_cast<const f32x4*>(a.odense + (size_t)hs * N * D + (size_t)p * D + col);
            const f32x4 r = od - o;
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.residual) + hoff + (size_t)p * D + col) =
                make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
          } else {
            f32x4* rp = reinterpret_cast<f32x4*>(static_cast<float*>(a.residual) + hoff + (size_t)p * D + col);
            *rp = *rp - o;
          }
        }
      }
    }
  }  // MODE != MODE_SCORE
  if constexpr (MODE != MODE_SCORE) return;

  // ---- key-score pass (selection): per-group key scores
  // c(j) = sum_i exp(s_ij - lse_i), from the rows' log-sum-exp that the
  // selection's dense pass left in a.lse.  It is a launch of its own so that
  // its registers hold only QK^T operands and scores: 64 query rows per wave
  // (each K operand read feeds twice the MFMAs, and a group of 64 needs no
  // cross-wave sum) at three waves per SIMD, where the dense pass runs two.
  // Only K is needed, so a stage holds two K tiles (2 BK keys) and the
  // barrier, the reduction through LDS and the flush to global memory come
  // once per 2 BK keys; the two halves are scored one after the other.
  float nlse[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = row0 + RPW * w + 16 * rb + 4 * lq + i;
      nlse[rb][i] = p < N ? -a.lse[(size_t)hs * N + p] : -INFINITY;
    }

  constexpr int BK2 = 2 * BK;
  const int nt2 = (N + BK2 - 1) / BK2;
  const int per = (nt2 + kchunks - 1) / kchunks;  // super-tiles per key range
  const int jbeg = min(nt2, kc * per), jend = min(nt2, jbeg + per);
  const int wpg = a.G / RPW;  // waves per group
  const int gpt = BM / a.G;   // groups per tile
  auto issue_k2 = [&](char* stage, int jj) {  // keys jj*BK2 .. +BK2-1 into both halves of a stage
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
      const int ii = w + NW * u;
      const int t = ii * GE::RPI + lane / GE::CPR;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r = jj * BK2 + half * BK + t;
        const int row = r < N - 1 ? r : N - 1;
        const int off = (row * GE::ROWB) | chunk_off[u];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(stage + half * GE::TILE + ii * 1024), 16, off, 0, 0, 0);
      }
    }
  };
  auto flush = [&](int jj) {  // cross-wave sums of super-tile jj -> colsum
    for (int t = tid; t < gpt * BK2; t += NW * 64) {
      const int gi = t / BK2, col = t % BK2, tok = jj * BK2 + col;
      const int g = row0 / a.G + gi;
      if (tok < N && g < a.ng) {
        float sum = 0.f;
        for (int ww = 0; ww < wpg; ++ww) sum += red[jj & 1][gi * wpg + ww][col];
        a.colsum[((size_t)hs * a.ng + g) * a.ldc + tok] = sum;
      }
    }
  };
  auto score_tile = [&](int jj, const char* cur, char* nxt) {
    wait_vm<0>();
    __syncthreads();
    if (jj + 1 < jend) issue_k2(nxt, jj + 1);
    if (jj > jbeg) flush(jj - 1);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const char* kt = cur + half * GE::TILE;
      bf16x8 kf[KK][TB];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) kf[kk][tb] = kfrag(kt, tb, kk);
      // S[row][token]: lane holds rows 16 rb + 4 lq + i of token 16 tb + lr
      f32x4 s[RB][TB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) s[rb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            s[rb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[rb][kk], kf[kk][tb], s[rb][tb], 0, 0, 0);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        float cs = 0.f;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(fmaf(s[rb][tb][i], sl2, nlse[rb][i]));
            cs = (rb == 0 && i == 0) ? p : cs + p;
          }
        cs = quad_rows_sum(cs);
        if (lq == 0) red[jj & 1][w][half * BK + 16 * tb + lr] = cs;
      }
    }
  };
  if (jend > jbeg) issue_k2(st0, jbeg);
  for (int jj = jbeg; jj < jend; jj += 2) {
    score_tile(jj, st0, st1);
    if (jj + 1 < jend) score_tile(jj + 1, st1, st0);
  }
  __syncthreads();
  if (jend > jbeg) flush(jend - 1);
}

// KV tile size: 32 tokens at d = 128 (the batched K and V operand reads of a
// 64-token tile would not fit the register budget), 64 tokens at d = 64.
template <int D>
constexpr int tile_tokens() {
  return D == 128 ? 32 : 64;
}

template <int D, int NW, int MODE>
hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  constexpr int BM = NW * (MODE == MODE_SCORE ? 64 : 32);
  const int tiles = (MODE == MODE_REUSE || MODE == MODE_RESINIT) ? a.ng : (a.N + BM - 1) / BM;
  AttnArgs b = a;
  b.kchunks = 1;
  if constexpr (MODE == MODE_SCORE) {
    // Enough work items for the last of the rounds of resident workgroups
    // to be a small part of the launch.
    const long long items = (long long)a.nheads * tiles;
    const int nt2 = (a.N + 2 * tile_tokens<D>() - 1) / (2 * tile_tokens<D>());
    if (items > 0) b.kchunks = (int)std::max<long long>(1, std::min<long long>(nt2, (kScoreItems + items - 1) / items));
  }
  const long long nblocks = (long long)a.nheads * tiles * b.kchunks;
  if (nblocks == 0) return hipSuccess;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_bf16_kernel<D, NW, MODE, tile_tokens<D>()>), dim3((unsigned)nblocks), dim3(NW * 64), 0,
                     s, b);
  return launched(s);
}

template <int D>
hipError_t launch_d(int mode, const AttnArgs& a, hipStream_t s) {
  switch (mode) {
    case MODE_PLAIN: return launch_one<D, 4, MODE_PLAIN>(a, s);
    case MODE_SELECT: return launch_one<D, 4, MODE_SELECT>(a, s);
    case MODE_SCORE: return launch_one<D, 4, MODE_SCORE>(a, s);
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
