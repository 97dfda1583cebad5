/*
 * A plain C99 client of the C ABI in include/mcs.h: it calls the host-only
 * entry points (version, status strings, metadata layout and sizes) and the
 * argument checks that fail before any device work, so it runs without a
 * GPU.  Exit status 0 means every check held; otherwise the first failed
 * check is printed.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mcs.h"

static int failures = 0;

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  mcs_attn_desc d;
  mcs_meta m;
  int32_t keep[3] = {64, 100, 7};
  size_t bytes, ws1, ws3;
  uint64_t end;

  CHECK(mcs_version() == MCS_VERSION);
  CHECK(strcmp(mcs_status_string(MCS_SUCCESS), "MCS_SUCCESS") == 0);
  CHECK(strcmp(mcs_status_string(MCS_ERROR_META_MISMATCH), "MCS_ERROR_META_MISMATCH") == 0);
  CHECK(mcs_last_hip_error() == 0);

  /* three heads of 1000 tokens, d = 64, bf16, groups of 64 */
  d.num_heads = 3;
  d.seq_len = 1000;
  d.head_dim = 64;
  d.dtype = MCS_DTYPE_BF16;
  d.softmax_scale = 0.0f;
  memset(&m, 0, sizeof m);
  CHECK(mcs_meta_layout(&d, 64, keep, &m) == MCS_SUCCESS);
  CHECK(m.version == MCS_META_VERSION);
  CHECK(m.num_groups == 16);                       /* ceil(1000 / 64) */
  CHECK(m.max_keep == 100);
  CHECK(m.total_idx == 16 * (64 + 100 + 7));
  CHECK(m.base == NULL);
  CHECK(m.off_perm % 256 == 0 && m.off_count % 256 == 0 && m.off_order % 256 == 0 && m.off_idx % 256 == 0 &&
        m.off_residual % 256 == 0);
  CHECK(m.off_order >= m.off_count + (uint64_t)3 * 16 * 4 && m.off_idx >= m.off_order + (uint64_t)3 * 16 * 4);
  CHECK(m.residual_dtype == MCS_DTYPE_FP32);
  end = m.off_residual + (uint64_t)3 * 1000 * 64 * 4; /* float32 residual [H][N][d] */
  CHECK(m.bytes >= end);
  bytes = mcs_meta_bytes(&d, 64, keep);
  CHECK(bytes == m.bytes);
  /* the same layout with a bf16 residual */
  CHECK(mcs_meta_layout_ex(&d, 64, keep, MCS_DTYPE_BF16, &m) == MCS_SUCCESS);
  CHECK(m.residual_dtype == MCS_DTYPE_BF16 && m.bytes == end - (uint64_t)3 * 1000 * 64 * 2);

  ws1 = mcs_select_workspace_bytes(&d, 64, 1);
  ws3 = mcs_select_workspace_bytes(&d, 64, 3);
  CHECK(ws1 > 0 && ws3 > ws1);
  CHECK(mcs_select_workspace_bytes(&d, 64, 99) == ws3); /* clamped to H */
  {
    mcs_select_options o;
    memset(&o, 0, sizeof o);
    o.kv_block = 1;
    o.residual = 1;
    o.residual_dtype = MCS_DTYPE_BF16;
    CHECK(mcs_select_workspace_bytes_ex(&d, 64, 1, &o) == ws1 + (size_t)1000 * 64 * 4);
    CHECK(mcs_select_workspace_bytes_ex(&d, 64, 1, NULL) == ws1);
  }

  /* argument checks that fail before any device work */
  CHECK(mcs_meta_layout(&d, 32, keep, &m) == MCS_ERROR_UNSUPPORTED_SHAPE);
  keep[1] = 1001;
  CHECK(mcs_meta_layout(&d, 64, keep, &m) == MCS_ERROR_INVALID_VALUE);
  CHECK(mcs_meta_bytes(&d, 64, keep) == 0);
  keep[1] = 100;
  d.head_dim = 96;
  CHECK(mcs_meta_layout(&d, 64, keep, &m) == MCS_ERROR_UNSUPPORTED_SHAPE);
  d.head_dim = 64;
  d.seq_len = MCS_MAX_SEQ_LEN + 1;
  CHECK(mcs_meta_layout(&d, 64, keep, &m) == MCS_ERROR_UNSUPPORTED_SHAPE);
  d.seq_len = 1000;
  CHECK(mcs_dense_attn(&d, NULL, NULL, NULL, NULL, NULL) == MCS_ERROR_INVALID_VALUE);
  CHECK(mcs_sparse_attn(NULL, NULL, NULL, NULL, NULL, NULL, NULL) == MCS_ERROR_INVALID_VALUE);
  /* the row top-k validates sizes, strides and buffers before any device call */
  {
    float* fake = (float*)(uintptr_t)0x1000;     /* never dereferenced: every call below fails validation */
    int32_t* fidx = (int32_t*)(uintptr_t)0x2000;
    CHECK(mcs_topk_rows(fake, 8, 0, 8, 2, fidx, NULL) == MCS_SUCCESS);        /* no rows: nothing to do */
    CHECK(mcs_topk_rows(NULL, 8, 1, 8, 2, fidx, NULL) == MCS_ERROR_INVALID_VALUE);
    CHECK(mcs_topk_rows(fake, 8, 1, 8, 2, NULL, NULL) == MCS_ERROR_INVALID_VALUE);
    CHECK(mcs_topk_rows(fake, 8, 1, 8, 0, fidx, NULL) == MCS_ERROR_INVALID_VALUE);   /* k < 1 */
    CHECK(mcs_topk_rows(fake, 8, 1, 8, 9, fidx, NULL) == MCS_ERROR_INVALID_VALUE);   /* k > n */
    CHECK(mcs_topk_rows(fake, 6, 1, 6, 2, fidx, NULL) == MCS_ERROR_INVALID_VALUE);   /* ld not a multiple of 4 */
    CHECK(mcs_topk_rows(fake, 4, 1, 8, 2, fidx, NULL) == MCS_ERROR_INVALID_VALUE);   /* ld < n */
    CHECK(mcs_topk_rows(fake, 8, -1, 8, 2, fidx, NULL) == MCS_ERROR_INVALID_VALUE);  /* rows < 0 */
    CHECK(mcs_topk_rows(fake, 8, 1, 0, 1, fidx, NULL) == MCS_ERROR_INVALID_VALUE);   /* n < 1 */
    CHECK(mcs_topk_rows((float*)((char*)fake + 4), 8, 1, 8, 2, fidx, NULL) == MCS_ERROR_MISALIGNED);
    CHECK(mcs_topk_rows(fake, 8, 1, 8, 2, (int32_t*)((char*)fidx + 2), NULL) == MCS_ERROR_MISALIGNED);
  }

  if (failures == 0) printf("C ABI host calls: all checks held\n");
  return failures == 0 ? 0 : 1;
}
