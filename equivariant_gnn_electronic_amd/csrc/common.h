// Internal helpers shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstddef>

#include "egnn.h"

namespace egnn {

// ---- error reporting (thread-local text, see egnn_last_error) ----
void set_error(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

#define EGNN_TRY_HIP(expr)                                                        \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess) {                                                       \
      ::egnn::set_error("%s failed: %s", #expr, hipGetErrorString(e_));           \
      return EGNN_E_HIP;                                                          \
    }                                                                             \
  } while (0)

#define EGNN_CHECK_LAUNCH()                                                       \
  do {                                                                            \
    hipError_t e_ = hipGetLastError();                                            \
    if (e_ != hipSuccess) {                                                       \
      ::egnn::set_error("kernel launch failed at %s:%d: %s", __FILE__, __LINE__,  \
                        hipGetErrorString(e_));                                   \
      return EGNN_E_HIP;                                                          \
    }                                                                             \
  } while (0)

#define EGNN_REQUIRE(cond, ...)                                                   \
  do {                                                                            \
    if (!(cond)) {                                                                \
      ::egnn::set_error(__VA_ARGS__);                                             \
      return EGNN_E_ARG;                                                          \
    }                                                                             \
  } while (0)

// ---- bf16 storage (raw 16-bit patterns; round to nearest even) ----
__host__ __device__ inline float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even.  On the device the conversion compiles to the gfx950
// v_cvt_pk_bf16_f32 instruction; the host version is the same rounding on
// the bits (finite values).
__host__ __device__ inline uint16_t f32_to_bf16(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
#else
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
#endif
}

template <typename T> struct Store;
template <> struct Store<float> {
  __device__ static inline float ld(const float *p) { return *p; }
  __device__ static inline void st(float *p, float v) { *p = v; }
};
template <> struct Store<uint16_t> {
  __device__ static inline float ld(const uint16_t *p) { return bf16_to_f32(*p); }
  __device__ static inline void st(uint16_t *p, float v) { *p = f32_to_bf16(v); }
};

// LDS writes and reads of one wave execute in issue order; this only keeps
// the compiler from moving LDS accesses across the point (no memory wait).
__device__ inline void wave_lds_order() {
  __builtin_amdgcn_wave_barrier();
  __asm__ volatile("" ::: "memory");
}

__host__ __device__ constexpr int cmin(int a, int b) { return a < b ? a : b; }
__host__ __device__ constexpr int cabs(int a) { return a < 0 ? -a : a; }

// Offset (in floats) of the degree-l block in the stored Wigner rows:
// rows m = -min(l,mmax)..min(l,mmax), columns m' = -l..l.
__host__ __device__ constexpr int d_block_offset(int l, int mmax) {
  int o = 0;
  for (int j = 0; j < l; ++j) o += (2 * cmin(j, mmax) + 1) * (2 * j + 1);
  return o;
}
__host__ __device__ constexpr int d_count(int lmax, int mmax) { return d_block_offset(lmax + 1, mmax); }

// Number of kept edge-frame coefficients (|m| <= mmax).
__host__ __device__ constexpr int kept_count(int lmax, int mmax) {
  int n = 0;
  for (int l = 0; l <= lmax; ++l) n += 2 * cmin(l, mmax) + 1;
  return n;
}
__host__ __device__ constexpr int pair_count(int lmax, int mmax) {
  int n = 0;
  for (int m = 0; m <= mmax; ++m) n += lmax - m + 1;
  return n;
}
// index of gate pair (m, l), m = 0..mmax, l = m..lmax
__host__ __device__ constexpr int pair_index(int m, int l, int lmax) {
  int p = 0;
  for (int j = 0; j < m; ++j) p += lmax - j + 1;
  return p + (l - m);
}

// Shapes of one layer, computed on the host and passed to kernels by value.
struct LayerShape {
  int lmax, mmax, C, n_rbf;
  int K;            // (lmax+1)^2
  int n_pairs;      // radial gate pairs
  int nD;           // stored Wigner entries per edge
  int gstride;      // floats per edge in geom
  int kept;         // kept coefficients K'
  // GEMM operand widths per |m| (m = 0..mmax): A_m [E][Kg[m]], Y_m [E][Ng[m]]
  int Kg[3], Ng[3];
  float r_cut;
  int storage;      // egnn_dtype
};

bool make_shape(const egnn_layer_desc *d, LayerShape *s);

// Launch helpers
inline unsigned ceil_div(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

// (lmax, mmax) dispatch shared with the layer kernels
#define EGNN_DISPATCH_LM(lmax, mmax, FN, ...)                                     \
  switch ((lmax) * 10 + (mmax)) {                                                 \
    case 10: FN<1, 0>(__VA_ARGS__); break;                                        \
    case 11: FN<1, 1>(__VA_ARGS__); break;                                        \
    case 20: FN<2, 0>(__VA_ARGS__); break;                                        \
    case 21: FN<2, 1>(__VA_ARGS__); break;                                        \
    case 22: FN<2, 2>(__VA_ARGS__); break;                                        \
    case 30: FN<3, 0>(__VA_ARGS__); break;                                        \
    case 31: FN<3, 1>(__VA_ARGS__); break;                                        \
    case 32: FN<3, 2>(__VA_ARGS__); break;                                        \
    case 40: FN<4, 0>(__VA_ARGS__); break;                                        \
    case 41: FN<4, 1>(__VA_ARGS__); break;                                        \
    case 42: FN<4, 2>(__VA_ARGS__); break;                                        \
    case 60: FN<6, 0>(__VA_ARGS__); break;                                        \
    case 61: FN<6, 1>(__VA_ARGS__); break;                                        \
    case 62: FN<6, 2>(__VA_ARGS__); break;                                        \
    case 80: FN<8, 0>(__VA_ARGS__); break;                                        \
    case 81: FN<8, 1>(__VA_ARGS__); break;                                        \
    case 82: FN<8, 2>(__VA_ARGS__); break;                                        \
    default: break;                                                               \
  }

}  // namespace egnn
