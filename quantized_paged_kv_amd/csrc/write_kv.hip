// Quantise-on-write: rotate, group norms, nearest codebook level, pack, and
// scatter rows into persistent pages through a slot mapping.
//
// [D "Serving Route Design"]: the serving route writes packed rows into
// persistent pages; block = slot / block_size, offset = slot % block_size.
// [D "Recipe Strategy"]: each channel group stores its indices and a vector
// norm.  [T "Highlights"]: random Hadamard rotation before the codebook.
//
// Every floating-point step is float64 in a fixed order, with no fused
// multiply-add (this translation unit is built with -ffp-contract=off and the
// pragma below), so the bytes match any implementation that performs the same
// correctly rounded operations:
//   Walsh-Hadamard butterflies h = 1, 2, ..., d/2 (pair (j, j+h) -> a+b, a-b);
//   sum of squares by the pairwise tree over each group's listed channels
//   (adjacent pairs first);  sqrt and division correctly rounded;  fp64 ->
//   fp16 rounded to nearest even directly from fp64.
//
// Thread layout: one row (token, kv head, tensor) per D/8 lanes, eight
// channels per lane (lane L holds channels 8L..8L+7 after the load); a
// workgroup takes consecutive tokens of one kv head.  The butterflies for
// h < 8 run inside a lane, the rest across lanes (DPP).
#pragma clang fp contract(off)

#include <algorithm>
#include <type_traits>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kThreads = 256;

struct WriteParams {
  const void* src[2];   // K and V rows [T][H][D]
  uint8_t* pages[2];
  DevFormat fmt[2];
  const int64_t* slots;
  int64_t num_tokens;   // T
  int64_t num_units;    // ceil(T / rows per unit) * H
  int64_t num_slots;    // num_blocks * 16
  int32_t H;
  int32_t* dev_err;
};

template <int D, bool F32>
__global__ __launch_bounds__(kThreads, 5) void write_kv_kernel(WriteParams p) {
  constexpr int LPR = D / 8;              // lanes per row
  constexpr int RPB = kThreads / LPR;     // rows per block
  __shared__ double lds_w[RPB][D];
  __shared__ uint32_t lds_row[RPB][D / 8 + 1];  // packed row (<= D/2 bytes)
  // per bucket: the threshold inside it (+inf if none) and the count of
  // thresholds below it, one 16-byte entry (one LDS read per value)
  struct alignas(16) Bucket {
    double thr;
    uint32_t below, pad;
  };
  __shared__ Bucket lds_bk[2][256];

  __shared__ DevFormat sf;

  const int tensor = blockIdx.y;
  // the tensor's format to LDS once: reads of the argument block indexed by
  // the tensor would otherwise be vector loads inside the loop, which every
  // wait on the prefetched rows would also wait for
  {
    static_assert(sizeof(DevFormat) % 4 == 0, "format copied in words");
    const uint32_t* src = reinterpret_cast<const uint32_t*>(&p.fmt[tensor]);
    for (int i = threadIdx.x; i < (int)(sizeof(DevFormat) / 4); i += kThreads)
      reinterpret_cast<uint32_t*>(&sf)[i] = src[i];
  }
  __syncthreads();
  const DevFormat& f = sf;
  // bucket table of each group (bucket k spans z in [(k - off) / 32, (k + 1 - off) / 32))
  for (int g = 0; g < f.ng; ++g) {
    const int nthr = (1 << f.bits[g]) - 1;
    if (f.fast[g]) {
      const int k = threadIdx.x;   // kThreads == 256 buckets
      const double lo = ((double)k - (double)f.lut_off[g]) / 32.0, hi = lo + 1.0 / 32.0;
      int below = 0, inside = 0;
      for (int i = 0; i < nthr; ++i) {
        below += f.thr[g][i] < lo ? 1 : 0;
        inside |= (f.thr[g][i] >= lo && f.thr[g][i] < hi) ? 1 : 0;
      }
      lds_bk[g][k].thr = inside ? f.thr[g][below] : __builtin_inf();
      lds_bk[g][k].below = (uint32_t)below;
    }
  }
  __syncthreads();
  const int L = threadIdx.x % LPR;
  const int lr = threadIdx.x / LPR;
  // unit -> RPB consecutive tokens of one kv head: with the usual slot
  // mappings those rows fill whole tiles, so their partial-line writes meet
  // in one L2 and leave it as whole lines.  Workgroups loop over units so
  // that the set-up above is paid once per workgroup.
  // The loads of the next unit (its rows and slots) are issued before the
  // current unit is computed.
  struct Fetch {
    uint4 a, b;      // the lane's 8 channels (bf16: a only)
    int64_t slot;
  };
  // unit = blockIdx.x + i gridDim.x = tg H + head, stepped without dividing
  const uint32_t H = (uint32_t)p.H;
  const uint32_t step_tg = gridDim.x / H, step_h = gridDim.x % H;
  auto fetch = [&](int64_t unit, int64_t tg, int head) -> Fetch {
    Fetch x;
    const int64_t tok = tg * RPB + lr;
    const int64_t token = (unit < p.num_units && tok < p.num_tokens) ? tok : 0;
    const int64_t rr = token * p.H + head;
    if (F32) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(p.src[tensor]) + rr * D + 8 * L);
      x.a = src[0];
      x.b = src[1];
    } else {
      x.a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.src[tensor]) + rr * D + 8 * L);
      x.b = uint4{0u, 0u, 0u, 0u};
    }
    x.slot = p.slots[token];
    return x;
  };
  int64_t tg = blockIdx.x / H;
  int head = (int)(blockIdx.x % H);
  Fetch nxt = fetch(blockIdx.x, tg, head);
  for (int64_t unit = blockIdx.x; unit < p.num_units; unit += gridDim.x) {
  const Fetch cur = nxt;
  const int64_t cur_tg = tg;
  const int cur_head = head;
  tg += step_tg;
  head += (int)step_h;
  if (head >= (int)H) {
    head -= (int)H;
    ++tg;
  }
  nxt = fetch(unit + gridDim.x, tg, head);
  const int64_t tok = cur_tg * RPB + lr;
  const bool in_range = tok < p.num_tokens;
  const int64_t token = in_range ? tok : 0;
  const int64_t slot = cur.slot;
  const bool slot_ok = slot >= 0 && slot < p.num_slots;
  if (in_range && !slot_ok && cur_head == 0 && L == 0 && tensor == 0) {
    record_error(p.dev_err, TQ_ERR_INDEX, (int32_t)token);
  }
  const bool valid = in_range && slot_ok;

  // ---- load eight channels and apply the signs (exact: the sign bits are
  // flipped in the input words before the conversion to fp64)
  double v[8];
  const uint32_t sb = (f.sign_bits[(8 * L) >> 5] >> ((8 * L) & 31)) & 0xFFu;
  if (F32) {
    const uint4 a = cur.a, b = cur.b;
    const uint32_t w8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (double)__uint_as_float(w8[e] ^ (((sb >> e) & 1u) << 31));
  } else {
    // sign bits 2 i and 2 i + 1 to bits 15 and 31 of word i (sb | sb << 15
    // puts them 15 - 2 i places below)
    const uint32_t spread = sb | (sb << 15);
    const uint4 raw = cur.a;
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = w4[i] ^ ((spread << (15 - 2 * i)) & 0x80008000u);
      v[2 * i] = (double)__uint_as_float(w << 16);
      v[2 * i + 1] = (double)__uint_as_float(w & 0xFFFF0000u);
    }
  }

  // ---- Walsh-Hadamard transform, butterflies h = 1, 2, 4 inside the lane
#pragma unroll
  for (int h = 1; h < 8; h *= 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((e & h) == 0) {
        const double a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
    }
  }
  // ---- h = 8: partner lane L ^ 1, moved by DPP (the lower lane keeps a + b,
  // the upper a - b, a being the lower lane's value; one fma with a factor
  // of +-1 is the add or the subtraction itself: the product is exact and
  // the sum is rounded once)
  {
    const double sgn = (L & 1) ? -1.0 : 1.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __builtin_fma(sgn, v[e], lane_xor_d<1>(v[e], L));
  }
  // ---- h = 16 .. D/2 inside the lane: the row goes through LDS once, lane
  // L then holding channels L + LPR e (channel bits 4 and up are bits of e),
  // and back (the row's lanes are in one wave: a wave-scope fence orders
  // the exchange)
  double* const wrow = lds_w[lr];
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // the previous row's reads are done
#pragma unroll
  for (int e = 0; e < 8; e += 2) *reinterpret_cast<double2*>(wrow + 8 * L + e) = double2{v[e], v[e + 1]};
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = wrow[L + LPR * e];
#pragma unroll
  for (int h = 16 / LPR; h < 8; h *= 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((e & h) == 0) {
        const double a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) wrow[L + LPR * e] = v[e];
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // ---- each group's channels in listed order: lane L takes listed
  // positions [E*L, E*L+E) of each group (E = 8 for one group, 4 for two).
  const int ng = f.ng;
  double wg[8];
  if (ng == 1) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const double2 t = *reinterpret_cast<const double2*>(wrow + 8 * L + e);
      wg[e] = t.x;
      wg[e + 1] = t.y;
    }
  } else {
    const int m = D / 2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int g = e >> 2;
      wg[e] = wrow[f.ch[g * m + 4 * L + (e & 3)]];
    }
  }

  // ---- sums of squares: the pairwise tree over each group
  double sq[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sq[e] = wg[e] * wg[e];
  const double s01 = sq[0] + sq[1], s23 = sq[2] + sq[3], s45 = sq[4] + sq[5], s67 = sq[6] + sq[7];
  const double s03 = s01 + s23, s47 = s45 + s67;
  double ss[2];
  if (ng == 1) {
    ss[0] = s03 + s47;
    ss[1] = 0.0;
  } else {
    ss[0] = s03;
    ss[1] = s47;
  }
  ss[0] = ss[0] + lane_xor_d<1>(ss[0], L);
  ss[0] = ss[0] + lane_xor_d<2>(ss[0], L);
  ss[0] = ss[0] + lane_xor_d<4>(ss[0], L);
  if constexpr (LPR == 16) ss[0] = ss[0] + lane_xor_d<8>(ss[0], L);
  if (ng == 2) {   // (uniform: the tensor's format)
    ss[1] = ss[1] + lane_xor_d<1>(ss[1], L);
    ss[1] = ss[1] + lane_xor_d<2>(ss[1], L);
    ss[1] = ss[1] + lane_xor_d<4>(ss[1], L);
    if constexpr (LPR == 16) ss[1] = ss[1] + lane_xor_d<8>(ss[1], L);
  }

  // ---- norms, thresholds, indices and the packed bit fields: group g
  // holds values wg[BASE .. BASE + E) (compile-time, so that every index
  // into the lane's arrays is static)
  uint32_t field[2] = {0u, 0u};
  uint16_t norm16[2] = {0, 0};
  auto quant = [&](auto gk, auto ek) {
    constexpr int g = decltype(gk)::value;
    constexpr int E = decltype(ek)::value;
    constexpr int BASE = g * E;
    const int bits = f.bits[g];
    const int levels = 1 << bits;
    const int m = D / (8 / E);   // channels of the group: D (one group) or D / 2
    const double s = ss[g];
    uint32_t fld = 0;
    if (s == 0.0) {
      const uint32_t z = (uint32_t)(levels / 2 - 1);
#pragma unroll
      for (int e = 0; e < E; ++e) fld |= z << (bits * e);
      norm16[g] = 0;
    } else {
      norm16[g] = f64_to_f16_rne(__builtin_sqrt(s / (double)D));
      const double r = __builtin_sqrt(s / (double)m);
      uint32_t idx[E];
      // idx = number of scaled thresholds T_i = thr_i * r below the value.
      // Fast path: the bucket of z = w / r (float estimate) gives the count
      // of thresholds in lower buckets, exact because no threshold lies
      // within the estimate's error of a bucket edge; the one threshold a
      // bucket may hold is compared exactly.  Otherwise every threshold is
      // compared (the level count made a compile-time constant so that the
      // comparisons unroll).
      // (the float estimate needs r inside the normal float range; |z| <= sqrt(m))
      if (f.fast[g] && r > 1e-30 && r < 1e30) {
        const float rinv = __builtin_amdgcn_rcpf((float)r);
        const float off = f.lut_off[g];
        // all buckets first, then all their entries (one LDS round trip)
        int kb[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float z = (float)wg[BASE + e] * rinv;
          const int k = __float2int_rd(__builtin_fmaf(z, 32.0f, off));
          kb[e] = k < 0 ? 0 : (k > 255 ? 255 : k);
        }
        Bucket ent[E];
#pragma unroll
        for (int e = 0; e < E; ++e) ent[e] = lds_bk[g][kb[e]];
        // the threshold inside the bucket, scaled (+inf when none: never below)
#pragma unroll
        for (int e = 0; e < E; ++e) idx[e] = ent[e].below + (ent[e].thr * r < wg[BASE + e] ? 1u : 0u);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) idx[e] = 0;
        auto count_below = [&](auto lv) {
          constexpr int LV = decltype(lv)::value;
          double T[LV - 1];
#pragma unroll
          for (int i = 0; i < LV - 1; ++i) T[i] = f.thr[g][i] * r;
#pragma unroll
          for (int i = 0; i < LV - 1; ++i)
#pragma unroll
            for (int e = 0; e < E; ++e) idx[e] += (T[i] < wg[BASE + e]) ? 1u : 0u;
        };
        if (levels == 16) count_below(std::integral_constant<int, 16>{});
        else if (levels == 8) count_below(std::integral_constant<int, 8>{});
        else count_below(std::integral_constant<int, 4>{});
      }
#pragma unroll
      for (int e = 0; e < E; ++e) fld |= idx[e] << (bits * e);
    }
    field[g] = fld;
  };
  if (ng == 1) {
    quant(std::integral_constant<int, 0>{}, std::integral_constant<int, 8>{});
  } else {
    quant(std::integral_constant<int, 0>{}, std::integral_constant<int, 4>{});
    quant(std::integral_constant<int, 1>{}, std::integral_constant<int, 4>{});
  }
  const int E = (ng == 1) ? 8 : 4;

  const int64_t blk = slot >> 4;
  const int offs = (int)(slot & 15);
  uint8_t* tile = p.pages[tensor] + ((int64_t)blk * p.H + cur_head) * f.tile_bytes;
  if (ng == 1) {
    // one group: lane L's eight indices are the row's bytes [bits L, bits
    // (L + 1)) -- a dword (4-bit), a half-word (2-bit) or three bytes -- and
    // go straight to their place in the index plane (row-major, or run
    // 16 (offs % 4) + byte / c, place offs / 4 of the lane-major plane)
    const int bits = f.bits[0];
    const uint32_t fld = field[0];
    const int b0 = bits * L;   // first row byte of this lane
    const int c = f.chunk;
    // (run, place) of a byte of the lane-major plane; the chunk of the
    // served one-group formats is a power of two (shifts, not a division)
    const bool c_pow2 = (c & (c - 1)) == 0;
    const int c_sh = __builtin_ctz((unsigned)c | 0x100u);
    auto at = [&](int byte) -> uint8_t* {
      if (c == 0) return tile + offs * f.row_bytes + byte;
      if (c_pow2)
        return tile + (((16 * (offs & 3) + (byte >> c_sh)) * 4 + (offs >> 2)) << c_sh) + (byte & (c - 1));
      return tile + ((16 * (offs & 3) + byte / c) * 4 + (offs >> 2)) * c + byte % c;
    };
    if (!valid) {
    } else if (bits == 4 && (c == 0 || c % 4 == 0)) {
      *reinterpret_cast<uint32_t*>(at(b0)) = fld;
    } else if (bits == 2 && (c == 0 || c % 2 == 0)) {
      *reinterpret_cast<uint16_t*>(at(b0)) = (uint16_t)fld;
    } else if (bits == 4 && c == 2) {
      *reinterpret_cast<uint16_t*>(at(b0)) = (uint16_t)fld;
      *reinterpret_cast<uint16_t*>(at(b0 + 2)) = (uint16_t)(fld >> 16);
    } else {
      for (int j = 0; j < bits; ++j) *at(b0 + j) = (uint8_t)(fld >> (8 * j));
    }
  } else {
  // ---- two groups: assemble the row in LDS, then store it with dword writes
  constexpr int WORDS = D / 8 + 1;
  for (int w = L; w < WORDS; w += LPR) lds_row[lr][w] = 0u;
  __syncthreads();
  for (int g = 0; g < ng; ++g) {
    const int bits = f.bits[g];
    const int nbits = E * bits;
    const int off = f.grp_byte_off[g] * 8 + E * L * bits;
    const int word = off >> 5, sh = off & 31;
    const uint32_t val = field[g];
    atomicOr(&lds_row[lr][word], val << sh);
    if (sh + nbits > 32) atomicOr(&lds_row[lr][word + 1], val >> (32 - sh));
  }
  __syncthreads();
  if (!valid) {
  } else if (f.octet) {
    // two-group V pages: octet o of group g (b bytes: 8 indices) goes to
    // run (m / 8) (offs % 4) + o of the group's sub-plane, place offs / 4;
    // lane L takes octet L % (m / 8) of group L / (m / 8)
    constexpr int OCT = D / 16;   // octets per group (m / 8, m = D / 2)
    const uint8_t* src = reinterpret_cast<const uint8_t*>(lds_row[lr]);
    for (int u = L; u < 2 * OCT; u += LPR) {
      const int g = u / OCT, o = u % OCT;
      const int b = f.bits[g];
      const int gbo = f.grp_byte_off[g];
      uint8_t* cd = tile + 16 * gbo + (OCT * (offs & 3) + o) * 4 * b + (offs >> 2) * b;
      const uint8_t* cs = src + gbo + o * b;
      if (b == 4) {
        *reinterpret_cast<uint32_t*>(cd) = (uint32_t)cs[0] | ((uint32_t)cs[1] << 8) | ((uint32_t)cs[2] << 16) |
                                           ((uint32_t)cs[3] << 24);
      } else if (b == 2) {
        *reinterpret_cast<uint16_t*>(cd) = (uint16_t)(cs[0] | (cs[1] << 8));
      } else {
        for (int k = 0; k < b; ++k) cd[k] = cs[k];
      }
    }
  } else if (f.chunk == 0) {   // row-major index plane
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + offs * f.row_bytes);
    for (int w = L; w < f.row_bytes / 4; w += LPR) dst[w] = lds_row[lr][w];
  } else {              // lane-major: chunk j of the row goes to run 16*(offs%4)+j, place offs/4
    const uint8_t* src = reinterpret_cast<const uint8_t*>(lds_row[lr]);
    const int c = f.chunk;
    for (int jj = L; jj < 16; jj += LPR) {
      uint8_t* cd = tile + ((16 * (offs & 3) + jj) * 4 + (offs >> 2)) * c;
      const uint8_t* cs = src + jj * c;
      if ((c & 3) == 0) {
        for (int w = 0; w < c / 4; ++w) reinterpret_cast<uint32_t*>(cd)[w] = reinterpret_cast<const uint32_t*>(cs)[w];
      } else if (c == 2) {
        *reinterpret_cast<uint16_t*>(cd) = *reinterpret_cast<const uint16_t*>(cs);
      } else {
        for (int b = 0; b < c; ++b) cd[b] = cs[b];
      }
    }
  }
  }
  if (valid && L == 0) {
    const int nslot = 4 * (offs & 3) + (offs >> 2);
    uint16_t* np = reinterpret_cast<uint16_t*>(tile + f.norm_off);
    for (int g = 0; g < ng; ++g) np[16 * g + nslot] = norm16[g];
  }
  }
}

// Workgroups of write_kv_kernel<D, F32> one CU holds at once (looked up
// once per instantiation).
template <int D, bool F32>
int resident_per_cu() {
  static const int n = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, write_kv_kernel<D, F32>, kThreads, 0) != hipSuccess ||
        b < 1)
      b = 1;
    return b;
  }();
  return n;
}

// The write path's fp64 operations on given inputs, as the write kernel
// compiles them (same file, same flags: no contraction): element i of each
// output is sqrt(a_i), a_i / b_i, a_i * b_i and the binary16 bits of a_i.
__global__ __launch_bounds__(256) void selftest_fp64_kernel(const double* a, const double* b, int64_t n,
                                                            double* out_sqrt, double* out_div, double* out_mul,
                                                            uint16_t* out_f16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const double x = a[i], y = b[i];
  out_sqrt[i] = __builtin_sqrt(x);
  out_div[i] = x / y;
  out_mul[i] = x * y;
  out_f16[i] = f64_to_f16_rne(x);
}

}  // namespace
}  // namespace tq

using namespace tq;

extern "C" tq_status tq_selftest_fp64(const double* a, const double* b, int64_t n, double* out_sqrt, double* out_div,
                                      double* out_mul, uint16_t* out_f16, tq_stream_t stream) {
  if (n < 0 || n >= (1ll << 31)) return set_error(TQ_ERR_VALUE, "n must be in [0, 2^31)");
  if (n == 0) return TQ_OK;
  if (!a || !b || !out_sqrt || !out_div || !out_mul || !out_f16) return set_error(TQ_ERR_VALUE, "NULL pointer");
  hipLaunchKernelGGL(selftest_fp64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), a, b, n, out_sqrt, out_div, out_mul, out_f16);
  return launch_status("tq_selftest_fp64 launch");
}

extern "C" tq_status tq_write_kv(const void* k, const void* v, tq_dtype in_dtype, int64_t num_tokens,
                                 int32_t num_kv_heads, const int64_t* slot_mapping, uint8_t* k_pages,
                                 uint8_t* v_pages, int64_t num_blocks, int32_t block_size,
                                 const tq_format* kfmt, const tq_format* vfmt, int32_t* dev_err,
                                 tq_stream_t stream) {
  if (!k && !v) return set_error(TQ_ERR_VALUE, "k and v are both NULL");
  if (in_dtype != TQ_BF16 && in_dtype != TQ_F32) return set_error(TQ_ERR_VALUE, "in_dtype must be BF16 or F32");
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0)
    return set_error(TQ_ERR_VALUE, "num_tokens must be >= 0, num_kv_heads and num_blocks > 0");
  if (block_size != TQ_BLOCK_SIZE) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "block_size must be 16");
  if (num_tokens > 0 && !slot_mapping) return set_error(TQ_ERR_VALUE, "slot_mapping is NULL");
  const void* src[2] = {k, v};
  uint8_t* pages[2] = {k_pages, v_pages};
  const tq_format* fmts[2] = {kfmt, vfmt};
  const char* names[2] = {"K", "V"};
  int d = 0;
  WriteParams p = {};
  int n_tensors = 0, first = -1;
  for (int t = 0; t < 2; ++t) {
    if (!src[t]) continue;
    tq_status st = check_format(fmts[t], names[t]);
    if (st != TQ_OK) return st;
    if (t == 1 && fmts[t]->qjl) return set_error(TQ_ERR_VALUE, "the QJL stage is defined for K formats only");
    if (t == 0 && fmts[t]->qjl && (reinterpret_cast<uintptr_t>(fmts[t]->qjl_proj) & 15))
      return set_error(TQ_ERR_VALUE, "qjl_proj must be 16-byte aligned");
    if (!pages[t]) return set_error(TQ_ERR_VALUE, std::string(names[t]) + " pages are NULL");
    if (d && fmts[t]->head_dim != d) return set_error(TQ_ERR_VALUE, "K and V head_dim differ");
    d = fmts[t]->head_dim;
    if (first < 0) first = t;
    p.src[n_tensors] = src[t];
    p.pages[n_tensors] = pages[t];
    make_dev_format(fmts[t], &p.fmt[n_tensors]);
    // V pages: octet runs per group for two-group formats, else a lane-major
    // index plane when the row bytes split into 16 runs
    if (t == 1 && p.fmt[n_tensors].ng == 2) p.fmt[n_tensors].octet = 1;
    else if (t == 1 && p.fmt[n_tensors].row_bytes % 16 == 0) p.fmt[n_tensors].chunk = p.fmt[n_tensors].row_bytes / 16;
    ++n_tensors;
  }
  if (num_tokens == 0) return TQ_OK;
  if (num_tokens * (int64_t)num_kv_heads >= (int64_t)1 << 40) return set_error(TQ_ERR_VALUE, "too many rows");
  p.slots = slot_mapping;
  p.num_tokens = num_tokens;
  p.num_slots = num_blocks * TQ_BLOCK_SIZE;
  p.H = num_kv_heads;
  p.dev_err = dev_err;
  const int rpb = kThreads / (d / 8);
  p.num_units = (num_tokens + rpb - 1) / rpb * num_kv_heads;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool f32 = in_dtype == TQ_F32;
  // persistent workgroups: as many as can be resident at once, every one
  // looping over units (a grid larger than that would run in rounds)
  auto launch = [&](auto dk, auto fk) {
    constexpr int DD = decltype(dk)::value;
    constexpr bool FF = decltype(fk)::value;
    const int64_t wgs = std::min<int64_t>(p.num_units, (int64_t)device_cus() * resident_per_cu<DD, FF>());
    hipLaunchKernelGGL((write_kv_kernel<DD, FF>), dim3((unsigned)wgs, (unsigned)n_tensors), dim3(kThreads), 0, s,
                       p);
  };
  using I128 = std::integral_constant<int, 128>;
  using I64 = std::integral_constant<int, 64>;
  if (d == 128) {
    if (f32) launch(I128{}, std::true_type{});
    else launch(I128{}, std::false_type{});
  } else {
    if (f32) launch(I64{}, std::true_type{});
    else launch(I64{}, std::false_type{});
  }
  tq_status st = launch_status("tq_write_kv launch");
  if (st != TQ_OK || !k || !kfmt->qjl) return st;
  QjlWriteArgs qa;
  qa.src = k;
  qa.f32 = f32;
  qa.pages = k_pages;
  qa.proj = kfmt->qjl_proj;
  qa.kappa = sqrt((double)kfmt->head_dim / (double)(kfmt->head_dim / kfmt->num_groups));
  qa.slots = slot_mapping;
  qa.num_tokens = num_tokens;
  qa.num_slots = p.num_slots;
  qa.H = num_kv_heads;
  return launch_qjl_write(qa, p.fmt[0], s);
}
