// C ABI of libmcs (declared in include/mcs.h): argument validation, the
// metadata and workspace layouts, and the launch sequence of the selection
// and reuse steps.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <vector>

#include "launch.h"
#include "mcs.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr uint64_t kAlign = 256;
#ifndef MCS_XCD_RUN
#define MCS_XCD_RUN 128
#endif
constexpr int kXcdRun = MCS_XCD_RUN;  // consecutive work items per XCD per round

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

mcs_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return MCS_ERROR_HIP;
}

mcs_status check_desc(const mcs_attn_desc* d) {
  if (!d) return MCS_ERROR_INVALID_VALUE;
  if (d->num_heads < 0 || d->seq_len < 0) return MCS_ERROR_INVALID_VALUE;
  if (d->head_dim != 64 && d->head_dim != 128) return MCS_ERROR_UNSUPPORTED_SHAPE;
  if (d->dtype != MCS_DTYPE_FP32 && d->dtype != MCS_DTYPE_BF16) return MCS_ERROR_UNSUPPORTED_SHAPE;
  if (d->seq_len > MCS_MAX_SEQ_LEN) return MCS_ERROR_UNSUPPORTED_SHAPE;
  if (!std::isfinite(d->softmax_scale)) return MCS_ERROR_INVALID_VALUE;
  return MCS_SUCCESS;
}

bool empty(const mcs_attn_desc* d) { return d->num_heads == 0 || d->seq_len == 0; }

float eff_scale(const mcs_attn_desc* d) {
  return d->softmax_scale > 0.f ? d->softmax_scale : (float)(1.0 / std::sqrt((double)d->head_dim));
}

mcs_status check_tensor(const void* p) {
  if (!p) return MCS_ERROR_INVALID_VALUE;
  if (!aligned(p, 16)) return MCS_ERROR_MISALIGNED;
  return MCS_SUCCESS;
}

mcs_status check_group_keep(const mcs_attn_desc* d, int32_t G, const int32_t* keep) {
  if (G != 64 && G != 128) return MCS_ERROR_UNSUPPORTED_SHAPE;
  if (d->num_heads > 0 && !keep) return MCS_ERROR_INVALID_VALUE;
  if (d->seq_len > 0)
    for (int h = 0; h < d->num_heads; ++h)
      if (keep[h] < 1 || keep[h] > d->seq_len) return MCS_ERROR_INVALID_VALUE;
  return MCS_SUCCESS;
}

// Region offsets and size of a metadata buffer holding `total` kept indices.
void place_regions(const mcs_attn_desc* d, int64_t total, mcs_meta* m) {
  const uint64_t H = (uint64_t)d->num_heads, N = (uint64_t)d->seq_len, D = (uint64_t)d->head_dim;
  uint64_t off = 0;
  m->off_perm = off;
  off = align_up(off + H * N * 4, kAlign);
  m->off_keep = off;
  off = align_up(off + H * 4, kAlign);
  m->off_idx_start = off;
  off = align_up(off + H * 8, kAlign);
  m->off_sched = off;
  off = align_up(off + H * 4, kAlign);
  m->off_idx = off;
  off = align_up(off + (uint64_t)total * 4, kAlign);
  m->off_residual = off;
  off = align_up(off + H * N * D * 4, kAlign);
  m->bytes = off;
}

void make_layout(const mcs_attn_desc* d, int32_t G, const int32_t* keep, mcs_meta* m) {
  const uint64_t H = (uint64_t)d->num_heads, N = (uint64_t)d->seq_len;
  std::memset(m, 0, sizeof(*m));
  m->version = MCS_META_VERSION;
  m->num_heads = d->num_heads;
  m->seq_len = d->seq_len;
  m->head_dim = d->head_dim;
  m->dtype = d->dtype;
  m->group_size = G;
  m->num_groups = (int32_t)((N + G - 1) / G);
  int64_t total = 0;
  int32_t mk = 0;
  if (N > 0)
    for (uint64_t h = 0; h < H; ++h) {
      total += (int64_t)m->num_groups * keep[h];
      mk = std::max(mk, keep[h]);
    }
  m->max_keep = mk;
  m->total_idx = total;
  place_regions(d, total, m);
}

uint64_t colsum_ld(int N) { return align_up((uint64_t)N, 64); }

// Leading dimension of the 64-key block scores of one score row.
uint64_t block_ld(int N) { return align_up((uint64_t)(N + 63) / 64, 64); }

struct WsLayout {
  uint64_t off_keys, off_proj, off_mean, off_colsum, per_head_colsum, per_head_block, per_head_lse, fixed;
};

// keys | projections | query means | key scores [hc][ng][ldc] | block scores [hc][ng][ldb] | row lse [hc][N]
WsLayout ws_layout(const mcs_attn_desc* d, int32_t G) {
  const uint64_t H = (uint64_t)d->num_heads, N = (uint64_t)d->seq_len;
  const uint64_t ng = (N + G - 1) / G;
  WsLayout w;
  w.off_keys = 0;
  w.off_proj = align_up(H * N, kAlign);
  w.off_mean = align_up(w.off_proj + (uint64_t)MCS_HASH_BITS * d->head_dim * 8, kAlign);
  w.off_colsum = align_up(w.off_mean + H * d->head_dim * 8, kAlign);
  w.per_head_colsum = ng * colsum_ld((int)N) * 4;
  w.per_head_block = ng * block_ld((int)N) * 4;
  w.per_head_lse = align_up(N * 4, kAlign);
  w.fixed = w.off_colsum;
  return w;
}

template <typename T>
T* at(void* base, uint64_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// Writes keep, idx_start and sched of a laid-out metadata buffer.
mcs_status upload_meta_tables(const mcs_meta* m, const int32_t* keep, hipStream_t s) {
  const int H = m->num_heads;
  std::vector<int64_t> start(H);
  std::vector<int32_t> sched(H);
  int64_t run = 0;
  for (int h = 0; h < H; ++h) {
    start[h] = run;
    run += (int64_t)m->num_groups * keep[h];
  }
  std::iota(sched.begin(), sched.end(), 0);
  std::stable_sort(sched.begin(), sched.end(), [&](int a, int b) { return keep[a] > keep[b]; });
  hipError_t e;
  if ((e = mcs::launch_fill_bytes(at<void>(m->base, m->off_keep), keep, (size_t)H * 4, s)) != hipSuccess)
    return hip_fail(e);
  if ((e = mcs::launch_fill_bytes(at<void>(m->base, m->off_idx_start), start.data(), (size_t)H * 8, s)) !=
      hipSuccess)
    return hip_fail(e);
  if ((e = mcs::launch_fill_bytes(at<void>(m->base, m->off_sched), sched.data(), (size_t)H * 4, s)) != hipSuccess)
    return hip_fail(e);
  return MCS_SUCCESS;
}

mcs::AttnArgs base_args(const mcs_attn_desc* d, const void* q, const void* k, const void* v) {
  mcs::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.H = d->num_heads;
  a.N = d->seq_len;
  a.D = d->head_dim;
  a.scale = eff_scale(d);
  a.run = kXcdRun;
  a.nheads = d->num_heads;
  return a;
}

hipError_t launch_attn(int dtype, int mode, const mcs::AttnArgs& a, hipStream_t s) {
  return dtype == MCS_DTYPE_BF16 ? mcs::launch_attn_bf16(mode, a, s) : mcs::launch_attn_f32(mode, a, s);
}

}  // namespace

extern "C" {

int mcs_version(void) { return MCS_VERSION; }

const char* mcs_status_string(mcs_status st) {
  switch (st) {
    case MCS_SUCCESS: return "MCS_SUCCESS";
    case MCS_ERROR_INVALID_VALUE: return "MCS_ERROR_INVALID_VALUE";
    case MCS_ERROR_UNSUPPORTED_SHAPE: return "MCS_ERROR_UNSUPPORTED_SHAPE";
    case MCS_ERROR_MISALIGNED: return "MCS_ERROR_MISALIGNED";
    case MCS_ERROR_BUFFER_TOO_SMALL: return "MCS_ERROR_BUFFER_TOO_SMALL";
    case MCS_ERROR_META_MISMATCH: return "MCS_ERROR_META_MISMATCH";
    case MCS_ERROR_HIP: return "MCS_ERROR_HIP";
  }
  return "MCS_UNKNOWN_STATUS";
}

int mcs_last_hip_error(void) { return g_last_hip_error; }

mcs_status mcs_dense_attn(const mcs_attn_desc* d, const void* q, const void* k, const void* v, void* o,
                          void* stream) {
  mcs_status st;
  if ((st = check_desc(d)) != MCS_SUCCESS) return st;
  if (empty(d)) return MCS_SUCCESS;
  for (const void* p : {q, k, v, (const void*)o})
    if ((st = check_tensor(p)) != MCS_SUCCESS) return st;
  mcs::AttnArgs a = base_args(d, q, k, v);
  a.o = o;
  const hipError_t e = launch_attn(d->dtype, mcs::MODE_PLAIN, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MCS_SUCCESS : hip_fail(e);
}

mcs_status mcs_meta_layout(const mcs_attn_desc* d, int32_t G, const int32_t* keep, mcs_meta* layout) {
  mcs_status st;
  if ((st = check_desc(d)) != MCS_SUCCESS) return st;
  if ((st = check_group_keep(d, G, keep)) != MCS_SUCCESS) return st;
  if (!layout) return MCS_ERROR_INVALID_VALUE;
  make_layout(d, G, keep, layout);
  return MCS_SUCCESS;
}

size_t mcs_meta_bytes(const mcs_attn_desc* d, int32_t G, const int32_t* keep) {
  mcs_meta m;
  if (mcs_meta_layout(d, G, keep, &m) != MCS_SUCCESS) return 0;
  return (size_t)m.bytes;
}

size_t mcs_select_workspace_bytes(const mcs_attn_desc* d, int32_t G, int32_t heads_per_chunk) {
  if (check_desc(d) != MCS_SUCCESS) return 0;
  if (G != 64 && G != 128) return 0;
  const WsLayout w = ws_layout(d, G);
  const int64_t hc = std::max<int64_t>(1, std::min<int64_t>(heads_per_chunk, std::max(1, d->num_heads)));
  return (size_t)(w.fixed + (uint64_t)hc * (w.per_head_colsum + w.per_head_block + w.per_head_lse));
}

mcs_status mcs_meta_init(const mcs_attn_desc* d, int32_t G, const int32_t* keep, void* meta_buf,
                         size_t meta_bytes, mcs_meta* meta_out, void* stream) {
  mcs_status st;
  if ((st = check_desc(d)) != MCS_SUCCESS) return st;
  if ((st = check_group_keep(d, G, keep)) != MCS_SUCCESS) return st;
  if (!meta_out) return MCS_ERROR_INVALID_VALUE;
  mcs_meta m;
  make_layout(d, G, keep, &m);
  if (!empty(d)) {
    if (!meta_buf) return MCS_ERROR_INVALID_VALUE;
    if (!aligned(meta_buf, kAlign)) return MCS_ERROR_MISALIGNED;
    if (meta_bytes < m.bytes) return MCS_ERROR_BUFFER_TOO_SMALL;
  }
  m.base = meta_buf;
  if (!empty(d) && (st = upload_meta_tables(&m, keep, static_cast<hipStream_t>(stream))) != MCS_SUCCESS) return st;
  *meta_out = m;
  return MCS_SUCCESS;
}

mcs_status mcs_select(const mcs_attn_desc* d, const void* q, const void* k, const void* v, int32_t G,
                      const int32_t* keep, const float* proj, void* meta_buf, size_t meta_bytes, void* ws,
                      size_t ws_bytes, void* o_dense_out, mcs_meta* meta_out, void* stream) {
  return mcs_select_ex(d, q, k, v, G, keep, proj, nullptr, meta_buf, meta_bytes, ws, ws_bytes, o_dense_out,
                       meta_out, stream);
}

mcs_status mcs_select_ex(const mcs_attn_desc* d, const void* q, const void* k, const void* v, int32_t G,
                         const int32_t* keep, const float* proj, const mcs_select_options* opts, void* meta_buf,
                         size_t meta_bytes, void* ws, size_t ws_bytes, void* o_dense_out, mcs_meta* meta_out,
                         void* stream) {
  mcs_status st;
  if ((st = check_desc(d)) != MCS_SUCCESS) return st;
  if ((st = check_group_keep(d, G, keep)) != MCS_SUCCESS) return st;
  if (!meta_out) return MCS_ERROR_INVALID_VALUE;
  mcs_select_options o{MCS_GROUPING_HASH, 1, 1, 0, 0, 0};
  if (opts) o = *opts;
  if ((o.grouping != MCS_GROUPING_HASH && o.grouping != MCS_GROUPING_RASTER &&
       o.grouping != MCS_GROUPING_CENTRED_HASH && o.grouping != MCS_GROUPING_MORTON) ||
      (o.kv_block != 1 && o.kv_block != 64) || (o.residual != 0 && o.residual != 1))
    return MCS_ERROR_INVALID_VALUE;
  if (o.grouping == MCS_GROUPING_MORTON) {
    for (int g : {o.grid_t, o.grid_y, o.grid_x})
      if (g < 1 || g > 1024) return MCS_ERROR_INVALID_VALUE;
    if ((int64_t)o.grid_t * o.grid_y * o.grid_x != d->seq_len) return MCS_ERROR_INVALID_VALUE;
  } else if (o.grid_t != 0 || o.grid_y != 0 || o.grid_x != 0) {
    return MCS_ERROR_INVALID_VALUE;
  }
  if (o.kv_block > 1) {
    if (d->seq_len % o.kv_block) return MCS_ERROR_UNSUPPORTED_SHAPE;
    for (int h = 0; h < d->num_heads; ++h)
      if (keep[h] % o.kv_block) return MCS_ERROR_UNSUPPORTED_SHAPE;
  }
  mcs_meta m;
  make_layout(d, G, keep, &m);
  m.base = meta_buf;
  if (empty(d)) {
    *meta_out = m;
    return MCS_SUCCESS;
  }
  for (const void* p : {q, k, v})
    if ((st = check_tensor(p)) != MCS_SUCCESS) return st;
  if (o_dense_out && !aligned(o_dense_out, 16)) return MCS_ERROR_MISALIGNED;
  if (!proj || !meta_buf || !ws) return MCS_ERROR_INVALID_VALUE;
  if (!aligned(meta_buf, kAlign) || !aligned(ws, kAlign)) return MCS_ERROR_MISALIGNED;
  if (meta_bytes < m.bytes) return MCS_ERROR_BUFFER_TOO_SMALL;
  const WsLayout wl = ws_layout(d, G);
  const uint64_t per_head = wl.per_head_colsum + wl.per_head_block + wl.per_head_lse;
  if (ws_bytes < wl.fixed + per_head) return MCS_ERROR_BUFFER_TOO_SMALL;
  const int H = d->num_heads, N = d->seq_len, D = d->head_dim;
  const int hc = (int)std::min<uint64_t>((uint64_t)H, (ws_bytes - wl.fixed) / per_head);
  hipStream_t s = static_cast<hipStream_t>(stream);

  if ((st = upload_meta_tables(&m, keep, s)) != MCS_SUCCESS) return st;
  std::vector<double> proj64((size_t)MCS_HASH_BITS * D);
  for (size_t i = 0; i < proj64.size(); ++i) proj64[i] = (double)proj[i];
  hipError_t e;
  double* dproj = at<double>(ws, wl.off_proj);
  uint8_t* keys = at<uint8_t>(ws, wl.off_keys);
  float* colsum = at<float>(ws, wl.off_colsum);
  float* bscore = at<float>(ws, wl.off_colsum + (uint64_t)hc * wl.per_head_colsum);
  float* lse = at<float>(ws, wl.off_colsum + (uint64_t)hc * (wl.per_head_colsum + wl.per_head_block));
  int32_t* perm = at<int32_t>(meta_buf, m.off_perm);
  if (o.grouping == MCS_GROUPING_HASH || o.grouping == MCS_GROUPING_CENTRED_HASH) {
    double* mean = nullptr;
    if (o.grouping == MCS_GROUPING_CENTRED_HASH) {
      mean = at<double>(ws, wl.off_mean);
      if ((e = mcs::launch_query_mean(q, d->dtype, mean, H, N, D, s)) != hipSuccess) return hip_fail(e);
    }
    if ((e = mcs::launch_fill_bytes(dproj, proj64.data(), proj64.size() * 8, s)) != hipSuccess) return hip_fail(e);
    if ((e = mcs::launch_hash_keys(q, d->dtype, dproj, mean, keys, H, N, D, s)) != hipSuccess) return hip_fail(e);
    if ((e = mcs::launch_perm_sort(keys, perm, H, N, s)) != hipSuccess) return hip_fail(e);
  } else if (o.grouping == MCS_GROUPING_MORTON) {
    if ((e = mcs::launch_morton_perm(perm, H, N, o.grid_t, o.grid_y, o.grid_x, s)) != hipSuccess) return hip_fail(e);
  } else if ((e = mcs::launch_iota_perm(perm, H, N, s)) != hipSuccess) {
    return hip_fail(e);
  }

  mcs::AttnArgs a = base_args(d, q, k, v);
  a.residual = at<float>(meta_buf, m.off_residual);
  a.colsum = colsum;
  a.lse = lse;
  a.perm = perm;
  a.keep = at<int32_t>(meta_buf, m.off_keep);
  a.idx_start = at<int64_t>(meta_buf, m.off_idx_start);
  a.sched = at<int32_t>(meta_buf, m.off_sched);
  a.idx = at<int32_t>(meta_buf, m.off_idx);
  a.G = G;
  a.ng = m.num_groups;
  a.total_idx = m.total_idx;
  a.ldc = (int)colsum_ld(N);
  for (int h0 = 0; h0 < H; h0 += hc) {
    a.head0 = h0;
    a.nheads = std::min(hc, H - h0);
    a.o = o_dense_out;
    if ((e = launch_attn(d->dtype, mcs::MODE_SELECT, a, s)) != hipSuccess) return hip_fail(e);
    if (d->dtype == MCS_DTYPE_BF16 && (e = launch_attn(d->dtype, mcs::MODE_SCORE, a, s)) != hipSuccess)
      return hip_fail(e);
    if (o.kv_block == 1) {
      e = mcs::launch_group_topk(colsum, a.ldc, at<int32_t>(meta_buf, m.off_idx), a.keep, a.idx_start, h0,
                                 a.nheads, a.ng, N, 1, s);
    } else {
      const int nb = N / o.kv_block, ldb = (int)block_ld(N);
      e = mcs::launch_block_scores(colsum, a.ldc, bscore, ldb, (long long)a.nheads * a.ng, nb, s);
      if (e == hipSuccess)
        e = mcs::launch_group_topk(bscore, ldb, at<int32_t>(meta_buf, m.off_idx), a.keep, a.idx_start, h0,
                                   a.nheads, a.ng, nb, o.kv_block, s);
    }
    if (e != hipSuccess) return hip_fail(e);
    a.o = nullptr;
    if (o.residual)
      e = launch_attn(d->dtype, mcs::MODE_RESINIT, a, s);
    else
      e = mcs::launch_zero_floats(a.residual + (size_t)h0 * N * D, (long long)a.nheads * N * D, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  *meta_out = m;
  return MCS_SUCCESS;
}

mcs_status mcs_sparse_attn(const mcs_attn_desc* d, const void* q, const void* k, const void* v,
                           const mcs_meta* m, void* o, void* stream) {
  mcs_status st;
  if ((st = check_desc(d)) != MCS_SUCCESS) return st;
  if (!m) return MCS_ERROR_INVALID_VALUE;
  if (m->version != MCS_META_VERSION || m->num_heads != d->num_heads || m->seq_len != d->seq_len ||
      m->head_dim != d->head_dim || m->dtype != d->dtype || (m->group_size != 64 && m->group_size != 128) ||
      m->num_groups != (d->seq_len + m->group_size - 1) / m->group_size)
    return MCS_ERROR_META_MISMATCH;
  // the regions must sit where this layout version puts them for the
  // struct's own index count (at most every head keeping every key)
  if (m->total_idx < 0 || (double)m->total_idx > (double)m->num_groups * d->seq_len * d->num_heads)
    return MCS_ERROR_META_MISMATCH;
  mcs_meta ref;
  place_regions(d, m->total_idx, &ref);
  if (m->off_perm != ref.off_perm || m->off_keep != ref.off_keep || m->off_idx_start != ref.off_idx_start ||
      m->off_sched != ref.off_sched || m->off_idx != ref.off_idx || m->off_residual != ref.off_residual ||
      m->bytes != ref.bytes)
    return MCS_ERROR_META_MISMATCH;
  if (empty(d)) return MCS_SUCCESS;
  for (const void* p : {q, k, v, (const void*)o})
    if ((st = check_tensor(p)) != MCS_SUCCESS) return st;
  if (!m->base) return MCS_ERROR_INVALID_VALUE;
  if (!aligned(m->base, kAlign)) return MCS_ERROR_MISALIGNED;
  mcs::AttnArgs a = base_args(d, q, k, v);
  a.o = o;
  a.residual = at<float>(m->base, m->off_residual);
  a.perm = at<int32_t>(m->base, m->off_perm);
  a.keep = at<int32_t>(m->base, m->off_keep);
  a.idx_start = at<int64_t>(m->base, m->off_idx_start);
  a.sched = at<int32_t>(m->base, m->off_sched);
  a.idx = at<int32_t>(m->base, m->off_idx);
  a.G = m->group_size;
  a.ng = m->num_groups;
  a.total_idx = m->total_idx;
  const hipError_t e = launch_attn(d->dtype, mcs::MODE_REUSE, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MCS_SUCCESS : hip_fail(e);
}

}  // extern "C"
