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
// channels per lane (lane L holds channels 8L..8L+7 after the load).  The
// butterflies for h < 8 run inside a lane, the rest across lanes.
#pragma clang fp contract(off)

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kThreads = 256;

struct WriteParams {
  const void* src[2];   // K and V rows [T][H][D]
  uint8_t* pages[2];
  DevFormat fmt[2];
  const int64_t* slots;
  int64_t num_rows;     // T * H
  int64_t num_slots;    // num_blocks * 16
  int32_t H;
  int32_t* dev_err;
};

__device__ __forceinline__ void record_error(int32_t* err, int32_t code, int32_t pos) {
  if (err && atomicCAS(err, 0, code) == 0) atomicExch(err + 1, pos);
}

template <int D, bool F32>
__global__ __launch_bounds__(kThreads) void write_kv_kernel(WriteParams p) {
  constexpr int LPR = D / 8;              // lanes per row
  constexpr int RPB = kThreads / LPR;     // rows per block
  __shared__ double lds_w[RPB][D];
  __shared__ uint32_t lds_row[RPB][D / 8 + 1];  // packed row (<= D/2 bytes)

  const int tensor = blockIdx.y;
  const DevFormat& f = p.fmt[tensor];
  const int L = threadIdx.x % LPR;
  const int lr = threadIdx.x / LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + lr;
  const bool in_range = row < p.num_rows;
  const int64_t rr = in_range ? row : 0;
  const int64_t token = rr / p.H;
  const int head = (int)(rr % p.H);
  const int64_t slot = p.slots[token];
  const bool slot_ok = slot >= 0 && slot < p.num_slots;
  if (in_range && !slot_ok && head == 0 && L == 0 && tensor == 0) {
    record_error(p.dev_err, TQ_ERR_INDEX, (int32_t)token);
  }
  const bool valid = in_range && slot_ok;

  // ---- load eight channels and apply the signs (exact)
  double v[8];
  if (F32) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(p.src[tensor]) + rr * D + 8 * L);
    const float4 a = src[0], b = src[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.src[tensor]) + rr * D + 8 * L);
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (double)__uint_as_float(w4[i] << 16);
      v[2 * i + 1] = (double)__uint_as_float(w4[i] & 0xFFFF0000u);
    }
  }
  {
    const uint32_t sb = (f.sign_bits[(8 * L) >> 5] >> ((8 * L) & 31)) & 0xFFu;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (sb & (1u << e)) v[e] = -v[e];
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
  // ---- h = 8, 16, ... across lanes: partner lane L ^ (h / 8)
#pragma unroll
  for (int k = 1; k < LPR; k *= 2) {
    const bool upper = (L & k) != 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double o = __shfl_xor(v[e], k);
      v[e] = upper ? (o - v[e]) : (v[e] + o);
    }
  }

  // ---- gather each group's channels in listed order: lane L takes listed
  // positions [E*L, E*L+E) of each group (E = 8 for one group, 4 for two).
  const int ng = f.ng;
  double wg[8];
  if (ng == 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) wg[e] = v[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) lds_w[lr][8 * L + e] = v[e];
    __syncthreads();
    const int m = D / 2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int g = e >> 2;
      wg[e] = lds_w[lr][f.ch[g * m + 4 * L + (e & 3)]];
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
#pragma unroll
  for (int k = 1; k < LPR; k *= 2) {
    ss[0] = ss[0] + __shfl_xor(ss[0], k);
    ss[1] = ss[1] + __shfl_xor(ss[1], k);
  }

  // ---- norms, thresholds, indices and the packed bit fields
  uint32_t field[2] = {0u, 0u};
  uint16_t norm16[2] = {0, 0};
  const int E = (ng == 1) ? 8 : 4;
  for (int g = 0; g < ng; ++g) {
    const int bits = f.bits[g];
    const int levels = 1 << bits;
    const int m = D / ng;
    const double s = ss[g];
    uint32_t fld = 0;
    if (s == 0.0) {
      const uint32_t z = (uint32_t)(levels / 2 - 1);
      for (int e = 0; e < E; ++e) fld |= z << (bits * e);
      norm16[g] = 0;
    } else {
      norm16[g] = f64_to_f16_rne(__builtin_sqrt(s / (double)D));
      const double r = __builtin_sqrt(s / (double)m);
      uint32_t idx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int i = 0; i < levels - 1; ++i) {
        const double t = (f16_bits_to_f64(f.cb[g][i]) + f16_bits_to_f64(f.cb[g][i + 1])) * 0.5;
        const double T = t * r;
#pragma unroll
        for (int e = 0; e < 8; ++e) idx[e] += (T < wg[e]) ? 1u : 0u;
      }
      const int base = (ng == 1) ? 0 : 4 * g;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < E) fld |= idx[base + e] << (bits * e);
    }
    field[g] = fld;
  }

  // ---- assemble the row in LDS, then store it with dword writes
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
  if (!valid) return;
  const int64_t blk = slot >> 4;
  const int offs = (int)(slot & 15);
  uint8_t* tile = p.pages[tensor] + ((int64_t)blk * p.H + head) * f.tile_bytes;
  if (f.chunk == 0) {   // row-major index plane
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
  if (L == 0) {
    const int nslot = 4 * (offs & 3) + (offs >> 2);
    uint16_t* np = reinterpret_cast<uint16_t*>(tile + f.norm_off);
    for (int g = 0; g < ng; ++g) np[16 * g + nslot] = norm16[g];
  }
}

}  // namespace
}  // namespace tq

using namespace tq;

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
    if (!pages[t]) return set_error(TQ_ERR_VALUE, std::string(names[t]) + " pages are NULL");
    if (d && fmts[t]->head_dim != d) return set_error(TQ_ERR_VALUE, "K and V head_dim differ");
    d = fmts[t]->head_dim;
    if (first < 0) first = t;
    p.src[n_tensors] = src[t];
    p.pages[n_tensors] = pages[t];
    make_dev_format(fmts[t], &p.fmt[n_tensors]);
    // V pages: lane-major index plane when the row bytes split into 16 runs
    if (t == 1 && p.fmt[n_tensors].row_bytes % 16 == 0) p.fmt[n_tensors].chunk = p.fmt[n_tensors].row_bytes / 16;
    ++n_tensors;
  }
  if (num_tokens == 0) return TQ_OK;
  if (num_tokens * (int64_t)num_kv_heads >= (int64_t)1 << 40) return set_error(TQ_ERR_VALUE, "too many rows");
  p.slots = slot_mapping;
  p.num_rows = num_tokens * num_kv_heads;
  p.num_slots = num_blocks * TQ_BLOCK_SIZE;
  p.H = num_kv_heads;
  p.dev_err = dev_err;
  const int rpb = kThreads / (d / 8);
  dim3 grid((unsigned)((p.num_rows + rpb - 1) / rpb), (unsigned)n_tensors);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool f32 = in_dtype == TQ_F32;
  if (d == 128) {
    if (f32) hipLaunchKernelGGL((write_kv_kernel<128, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((write_kv_kernel<128, false>), grid, dim3(kThreads), 0, s, p);
  } else {
    if (f32) hipLaunchKernelGGL((write_kv_kernel<64, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((write_kv_kernel<64, false>), grid, dim3(kThreads), 0, s, p);
  }
  return launch_status("tq_write_kv launch");
}
