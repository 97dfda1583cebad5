// Device-side helpers shared by the gfx950 kernels of libmcs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mcs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Logical block id with XCD locality.  The dispatcher hands workgroup b to XCD
// b % 8.  Inside each super-chunk of 8*run consecutive hardware ids, XCD x
// gets the `run` consecutive logical ids [x*run, (x+1)*run), so neighbouring
// work items (groups of one head) share an L2, while all XCDs still advance
// through the logical order together.  The tail that does not fill a whole
// super-chunk maps to itself.  The map is a bijection on [0, nblocks).
__device__ __forceinline__ int xcd_remap(int b, int nblocks, int run) {
  const int chunk = 8 * run;
  const int full = (nblocks / chunk) * chunk;
  if (b >= full) return b;
  const int s = b / chunk, r = b % chunk;
  return s * chunk + (r % 8) * run + r / 8;
}

// Clamps an index read from metadata into [0, n): metadata is a public layout
// that callers may fill themselves, so no value in it may lead a kernel out of
// bounds.
__device__ __forceinline__ int clamp_index(int i, int n) { return (unsigned)i < (unsigned)n ? i : (i < 0 ? 0 : n - 1); }

// Start and length of one group's kept keys: the group's slot of keep[h]
// indices starts at idx_start[h] + g * keep[h], and its first count[h][g]
// (clamped to [1, keep[h]]) are the kept keys; both kept inside [0, total).
__device__ __forceinline__ void group_keys(const int32_t* keep, const int64_t* idx_start, const int32_t* counts, int h,
                                           int g, int n, int ng, long long total, long long* start, int* count) {
  int k = keep[h];
  k = k < 1 ? 1 : (k > n ? n : k);
  long long s = idx_start[h] + (long long)g * k;
  if (s < 0 || s + k > total) {
    s = 0;
    if (k > total) k = (int)total;
  }
  int c = counts ? counts[(size_t)h * ng + g] : k;
  c = c < 1 ? 1 : (c > k ? k : c);
  *start = s;
  *count = c;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane value from lane (lane ^ mask) within the wave.
__device__ __forceinline__ float xor_shfl(float v, int mask) {
  const int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute(((lane ^ mask) << 2), __float_as_int(v)));
}

// Max / sum over the four lanes {l, l^16, l^32, l^48} (the four 16-lane rows
// of the wave), with the gfx950 row-swap permutes: each swap returns the
// lane's own value and its partner's, in some order.
__device__ __forceinline__ float quad_rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 t = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, t);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

}  // namespace mcs
