// Internal declarations shared by the libtq translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "tq.h"

namespace tq {

// ---------------------------------------------------------------- host side
tq_status set_error(tq_status st, const std::string& msg);
tq_status check_format(const tq_format* f, const char* which);
int row_index_bytes(const tq_format* f);
int mse_row_bytes(const tq_format* f);
int tile_bytes_of(const tq_format* f);
tq_status launch_status(const char* what);

// Device view of one format: everything a kernel needs, passed by value.
struct DevFormat {
  uint32_t sign_bits[4];   // bit j set <=> sign of channel j is -1
  uint16_t cb[2][16];      // fp16 codebooks per group
  uint8_t ch[128];         // listed channel order (group 0 then group 1)
  int32_t d, ng, m;        // head dim, groups, channels per group
  int32_t bits[2];
  int32_t grp_byte_off[2]; // byte offset of each group's bit string in a row
  int32_t row_bytes;       // index bytes per row
  int32_t tile_bytes;
  int32_t norm_off;        // byte offset of the norm plane in a tile
  int32_t chunk;           // V pages: bytes per lane run of the index plane (0: row-major)
  double thr[2][15];       // decision thresholds: midpoints of adjacent fp16 levels (exact)
  // Bucketed search for the level index (see the write kernel): bucket
  // k = floor(32 z + lut_off) of the scaled value z holds at most one
  // threshold, none within 2% of a bucket width of its edges, all inside
  // buckets 1..254; fast[g] = 0 when no offset meets that (then every
  // threshold is compared).
  float lut_off[2];
  int32_t fast[2];
  int32_t qjl;             // QJL stage: sign bits after the MSE bytes, residual norms after the norms
  int32_t sign_off;        // byte offset of the sign bits in a row (= MSE bytes)
  int32_t rnorm_off;       // byte offset of the residual-norm plane in a tile
  int32_t octet;           // V pages of two-group formats: index plane in octet runs per group
};

void make_dev_format(const tq_format* f, DevFormat* out);
int device_cus();

// QJL stage (qjl.hip): launched by tq_write_kv after the MSE write of the
// same rows, and by tq_decode_paged_multi for K formats with the stage.
struct QjlWriteArgs {
  const void* src;          // K rows [T][H][D]
  bool f32;
  uint8_t* pages;
  const float* proj;        // [ng][m][m]
  double kappa;             // sqrt(D / m), correctly rounded on the host
  const int64_t* slots;
  int64_t num_tokens, num_slots;
  int32_t H;
};
tq_status launch_qjl_write(const QjlWriteArgs& a, const DevFormat& kf, hipStream_t st);

struct QjlDecodeArgs {
  const void* q;
  bool q_f32;
  int32_t S, Hq, Hkv, G;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  int64_t num_blocks;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* context_lens;
  const float* proj;
  float scale;
  int32_t P;
  float* part_o;            // P > 1: [S][Hq][P][D] then lse [S][Hq][P]
  float* part_lse;
  void* out;
  bool out_f32;
  float* lse;
  int32_t* dev_err;
};
tq_status launch_qjl_decode(const QjlDecodeArgs& a, const DevFormat& kf, const DevFormat& vf, hipStream_t st);

// ------------------------------------------------------ host + device helpers

// IEEE binary16 bit pattern of a double, rounded to nearest, ties to even,
// directly from the double (no intermediate float32, so no double rounding).
__host__ __device__ inline uint16_t f64_to_f16_rne(double x) {
  union {
    double d;
    uint64_t u;
  } v;
  v.d = x;
  const uint64_t b = v.u;
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
  if (a >= 0x7FF0000000000000ull) {  // inf or nan
    return (uint16_t)(sign | 0x7C00u | (a > 0x7FF0000000000000ull ? 0x0200u : 0u));
  }
  const int e = (int)(a >> 52) - 1023;
  if (e >= 16) return (uint16_t)(sign | 0x7C00u);  // >= 65536: overflow
  const uint64_t m = (a & 0x000FFFFFFFFFFFFFull) | 0x0010000000000000ull;
  if (e >= -14) {  // normal binary16 range (rounding may carry into inf)
    const uint64_t q = m >> 42;              // 11 significant bits
    const uint64_t rem = m & ((1ull << 42) - 1);
    const uint64_t half = 1ull << 41;
    uint32_t h = ((uint32_t)(e + 15) << 10) + (uint32_t)(q & 0x3FFu);
    if (rem > half || (rem == half && (q & 1u))) h += 1;
    return (uint16_t)(sign | h);
  }
  // subnormal binary16: units of 2^-24; value = m * 2^(e-52)
  const int shift = 28 - e;  // >= 43
  if (shift > 63) return sign;  // far below 2^-25 (includes double subnormals)
  const uint64_t q = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  uint32_t h = (uint32_t)q;
  if (rem > half || (rem == half && (q & 1u))) h += 1;
  return (uint16_t)(sign | h);
}

__host__ __device__ inline double f16_bits_to_f64(uint16_t h) {
  const int e = (h >> 10) & 0x1F, f = h & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = f ? __builtin_nan("") : __builtin_inf();
  } else {
    v = ldexp((double)(1024 + f), e - 25);
  }
  return (h & 0x8000u) ? -v : v;
}

// ------------------------------------------------------ device helpers

// Device error word: the first reporter sets (code, position); later ones
// leave it as it is.
__device__ __forceinline__ void record_error(int32_t* err, int32_t code, int32_t pos) {
  if (err && atomicCAS(err, 0, code) == 0) atomicExch(err + 1, pos);
}

// float -> bfloat16 bit pattern, rounded to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// fp16 half HI of w as fp32, exactly (subnormals by their definition, so the
// result does not depend on the denormal mode)
template <int HI>
__device__ __forceinline__ float f16_exact(uint32_t w) {
  const uint32_t h = HI ? (w >> 16) : (w & 0xFFFFu);
  const float mag = (h & 0x7C00u) ? (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0x7FFFu))
                                  : (float)(int)(h & 0x3FFu) * 0x1p-24f;
  return (h & 0x8000u) ? -mag : mag;
}

// fp16 pair (x0 * n0, x1 * n1) from fp32 operands, each product rounded once
// to fp16
__device__ __forceinline__ uint32_t mul_f2(float x0, float n0, float x1, float n1) {
  uint32_t r = 0;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]" : "+v"(r) : "v"(x0), "v"(n0));
  asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]" : "+v"(r) : "v"(x1), "v"(n1));
  return r;
}

// x * (fp16 half HI of w) in one v_fma_mix, rounded once
template <int HI>
__device__ __forceinline__ float mul_h(float x, uint32_t w) {
  float r;
  if constexpr (HI) asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(w));
  else asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(w));
  return r;
}
// x * (fp16 half HI of w) + y
template <int HI>
__device__ __forceinline__ float fma_h(float x, uint32_t w, float y) {
  float r;
  if constexpr (HI) asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(w), "v"(y));
  else asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(w), "v"(y));
  return r;
}
// fp16 pair (x0 * half 0 of w, x1 * half 1 of w), each rounded once
__device__ __forceinline__ uint32_t mul_h2(float x0, float x1, uint32_t w) {
  uint32_t r = 0;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(r) : "v"(x0), "v"(w));
  asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(r) : "v"(x1), "v"(w));
  return r;
}
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2_t as_u16x2(uint32_t x) { return __builtin_bit_cast(u16x2_t, x); }
// fp16 bit pattern of 2^(15 - e), minus one, for e in [-1, 39]: V norms above
// it would make p * n_V * 2^e overflow fp16's range (e = -1: every finite
// fp16 is below the bound)
__device__ __forceinline__ uint32_t v_bound_m1(int e) {
  const int k = 15 - e;
  const uint32_t h = k >= 16 ? 0x7C00u : (k >= -14 ? (uint32_t)(k + 15) << 10 : 1u << (k + 24));
  return h - 1u;
}

// ------------------------------------------------------ device lane helpers

// Value of x in lane (lane ^ K), K a power of two below 64, without the
// LDS crossbar: DPP quad permutes for K = 1, 2, the half-row mirror (lane
// i <-> 7 - i) followed by the quad reversal (i <-> 3 - i) for K = 4, the
// 8-lane row rotation for K = 8, and the gfx950 row-swap permutes for K =
// 16, 32 (after swapping a value with itself, the partner's copy is the
// first result in the upper row of each pair and the second in the lower).
template <int K>
__device__ __forceinline__ float lane_xor(float x, int lane) {
  const int xi = __float_as_int(x);
  if constexpr (K == 1) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  } else if constexpr (K == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  } else if constexpr (K == 4) {
    const int m = __builtin_amdgcn_mov_dpp(xi, 0x141, 0xF, 0xF, true);           // row_half_mirror
    return __int_as_float(__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, true));    // quad_perm 3,2,1,0
  } else if constexpr (K == 8) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(xi, 0x128, 0xF, 0xF, true));  // row_ror 8
  } else if constexpr (K == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else {
    static_assert(K == 32, "lane_xor: K must be a power of two below 64");
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  }
}

// Double in lane (lane ^ K): the two 32-bit halves moved separately.
template <int K>
__device__ __forceinline__ double lane_xor_d(double x, int lane) {
  const uint64_t u = __double_as_longlong(x);
  const float lo = lane_xor<K>(__uint_as_float((uint32_t)u), lane);
  const float hi = lane_xor<K>(__uint_as_float((uint32_t)(u >> 32)), lane);
  return __longlong_as_double((long long)(((uint64_t)__float_as_uint(hi) << 32) | __float_as_uint(lo)));
}

}  // namespace tq
