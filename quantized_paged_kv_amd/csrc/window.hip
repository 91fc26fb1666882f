// Exact attention over a dense window of cached tokens (kept in bf16 or
// f32, not quantised), optionally merged by log-sum-exp with the result of
// the packed-page decode.
//
// [D "Format Strategy"] lists a recent dense window and the preservation of
// boundary tokens among the first serving policies, and [D "Data
// Ownership"] has the compressed cache own its recent windows next to the
// compressed blocks.  Neither says how the window is attended; the reading
// here: the window's tokens (the sequence's first few tokens and its most
// recent ones, in any order, since attention over a set of tokens does not
// depend on their order) are attended exactly, in the original domain, and
// the result is combined with the packed history's (o, lse) by the same
// log-sum-exp identity as the split merge:
//   lse = M + ln(e^{lse_h - M} + e^{lse_w - M}),
//   o   = e^{lse_h - lse} o_h + e^{lse_w - lse} o_w.
//
// One workgroup of 512 threads per (sequence, kv head).  The window is
// walked in chunks of T tokens, the chunk's K and V rows staged in LDS by
// coalesced 16-B loads that are all issued before any is waited for (the
// first chunk's even before the window length is known: those rows lie
// inside the buffer whatever the length), so a chunk costs one memory round
// trip; an online softmax runs across chunks.  bf16 rows (the serving case)
// take both contractions on the matrix cores (window_bf16_kernel); f32 rows
// take fp32 FMAs on the vector units (window_f32_kernel).
#include <cmath>

#include "tq_internal.h"
#include "window_item.h"

namespace tq {
namespace {

constexpr int kWinThreads = 512;
constexpr int kWinMaxG = 16;     // q heads per kv head


template <int D>
struct WinCfg {
  static constexpr int ESZ = 4;
  static constexpr int ROWB = D * ESZ;                                  // bytes of one K or V row
  static constexpr int T = (65536 / ROWB) < 256 ? (65536 / ROWB) : 256;   // tokens per chunk
  static constexpr int KPITCH = ROWB + 16;   // padded K row in LDS (row t starts 4 t banks further)
  static constexpr int PPR = ROWB / 16;      // 16-B pieces per row
  static constexpr int NPC = T * PPR / kWinThreads;   // pieces per thread per tensor
  static constexpr int NHS = kWinThreads / T;         // head sets in the score phase
  static constexpr int NTS = kWinThreads / (D / 2);   // token ranges in the P.V phase
  static constexpr int QW = D + 4;                    // q row (words) in LDS
};

// ---------------------------------------------------------------- f32 rows
// Chunks of T = 128 (d = 128) or 256 (d = 64) tokens:
//   scores  thread t takes token t % T and the q heads congruent to t / T, in
//           fp32 FMAs; q rows are read at wave-uniform LDS addresses
//           (broadcast);
//   softmax wave w takes q heads w, w + 8: chunk max, rescale factor,
//           p = 2^(s - m) written back, chunk sum;
//   P.V     thread i takes dims 2 (i % (d/2)), +1 and one of 512 / (d/2)
//           token ranges, for every q head, so each V element is read from
//           LDS once; the ranges' sums are added at the end.
// GMAX (4, 8 or 16) bounds the q heads per kv head: the loops over heads run
// to GMAX without guards (rows past G hold stale values that are never
// stored), so their LDS reads can be issued together.
template <int D, int GMAX>
__global__ __launch_bounds__(kWinThreads) void window_f32_kernel(WindowParams p) {
  using C = WinCfg<D>;
  constexpr int T = C::T;
  // K rows then V rows; at the end the P.V range sums
  __shared__ __attribute__((aligned(16))) uint8_t kvt[T * C::KPITCH + T * C::ROWB];
  uint8_t* const kt = kvt;
  uint8_t* const vt = kvt + T * C::KPITCH;
  __shared__ __attribute__((aligned(16))) float sc[GMAX * T];      // [head][token]: scores, then p
  __shared__ __attribute__((aligned(16))) float q_s[GMAX * C::QW];   // q rows (f32)
  __shared__ float s_m[GMAX], s_l[GMAX], s_a[GMAX], s_hl[GMAX];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x / p.Hkv, kvh = blockIdx.x % p.Hkv;
  const int G = p.G;
  const int h0 = kvh * G;   // first q head of this kv head
  const int64_t row_bytes = (int64_t)p.Hkv * C::ROWB;                                  // between tokens
  const int64_t seq_off = ((int64_t)s * p.cap * p.Hkv + kvh) * C::ROWB;                // token 0 of (s, kvh)
  const uint8_t* kg = static_cast<const uint8_t*>(p.k) + seq_off;
  const uint8_t* vg = static_cast<const uint8_t*>(p.v) + seq_off;

  // every load of the set-up is issued before any is waited for: first the
  // small ones (q words, history lse, window length), then the first chunk's
  // rows, so that using the small ones waits for them alone and the whole
  // set-up costs one memory round trip
  constexpr int QPT = (GMAX * D / 2 + kWinThreads - 1) / kWinThreads;   // q pairs per thread (at most)
  uint2 qv[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int i = tid + kWinThreads * j;
    qv[j] = uint2{0u, 0u};
    if (i < G * (D / 2)) {
      const int64_t off = ((int64_t)s * p.Hq + h0) * D + 2 * i;   // pair i of the G rows (rows are contiguous)
      if (p.q_f32) qv[j] = *reinterpret_cast<const uint2*>(static_cast<const float*>(p.q) + off);
      else qv[j].x = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.q) + off);
    }
  }
  const float hl_own = (tid < G && p.hist_lse) ? p.hist_lse[(int64_t)s * p.Hq + h0 + tid] : -INFINITY;
  int n = p.lens[s];

  // chunk rows -> registers: piece tid + 512 i is 16 B of token (piece / PPR);
  // the first chunk is requested before the length is known (its rows lie
  // inside the buffer whatever the length)
  uint4 kr[C::NPC], vr[C::NPC];
  {
    const int lim = p.cap < T ? p.cap : T;
#pragma unroll
    for (int i = 0; i < C::NPC; ++i) {
      const int pc = tid + kWinThreads * i;
      const int t = pc / C::PPR, c = pc % C::PPR;
      const int64_t off = (int64_t)t * row_bytes + 16 * c;
      kr[i] = t < lim ? *reinterpret_cast<const uint4*>(kg + off) : uint4{0u, 0u, 0u, 0u};
      vr[i] = t < lim ? *reinterpret_cast<const uint4*>(vg + off) : uint4{0u, 0u, 0u, 0u};
    }
  }

  // window length, clamped to [0, cap] (out-of-range lengths reported)
  if (n < 0 || n > p.cap) {
    if (tid == 0 && kvh == 0) record_error(p.dev_err, TQ_ERR_INDEX, -1 - s);
    n = n < 0 ? 0 : p.cap;
  }
  // q rows of the G heads -> LDS (f32); the history lse values are kept
  // before anything is written (out and lse may alias the history buffers)
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int i = tid + kWinThreads * j;
    if (i < G * (D / 2)) {
      const int g = i / (D / 2), dp = i % (D / 2);
      float2 x;
      if (p.q_f32) x = float2{__uint_as_float(qv[j].x), __uint_as_float(qv[j].y)};
      else x = float2{__uint_as_float(qv[j].x << 16), __uint_as_float(qv[j].x & 0xFFFF0000u)};
      q_s[g * C::QW + 2 * dp] = x.x;
      q_s[g * C::QW + 2 * dp + 1] = x.y;
    }
  }
  if (tid < G) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
    s_hl[tid] = hl_own;
  }

  // P.V slot of this thread: dims 2 dp, 2 dp + 1 of every head, token range ts
  const int dp = tid % (D / 2), ts = tid / (D / 2);
  float acc[GMAX][2];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) acc[g][0] = acc[g][1] = 0.f;

  for (int c0 = 0; c0 < n; c0 += T) {
    const int nc = (n - c0) < T ? (n - c0) : T;
    if (c0 > 0) __syncthreads();   // the previous chunk's rows and probabilities have been read
#pragma unroll
    for (int i = 0; i < C::NPC; ++i) {
      const int pc = tid + kWinThreads * i;
      const int t = pc / C::PPR, c = pc % C::PPR;
      if (t < nc) {
        *reinterpret_cast<uint4*>(kt + t * C::KPITCH + 16 * c) = kr[i];
        *reinterpret_cast<uint4*>(vt + t * C::ROWB + 16 * c) = vr[i];
      }
    }
    // the next chunk's rows are requested now: their round trip overlaps
    // this chunk's arithmetic
    if (c0 + T < n) {
#pragma unroll
      for (int i = 0; i < C::NPC; ++i) {
        const int pc = tid + kWinThreads * i;
        const int t = pc / C::PPR, c = pc % C::PPR;
        const int64_t off = (int64_t)(c0 + T + t) * row_bytes + 16 * c;
        if (c0 + T + t < n) {
          kr[i] = *reinterpret_cast<const uint4*>(kg + off);
          vr[i] = *reinterpret_cast<const uint4*>(vg + off);
        }
      }
    }
    __syncthreads();
    // -------- scores (base-2 domain): token t of the chunk, heads hs, hs + NHS, ...
    // (hs is uniform over a wave: T is a multiple of 64)
    {
      const int t = tid % T;
      const int hs = __builtin_amdgcn_readfirstlane(tid / T);
      constexpr int NH = (GMAX + C::NHS - 1) / C::NHS;
      float dot[NH];
#pragma unroll
      for (int j = 0; j < NH; ++j) dot[j] = 0.f;
      if (t < nc) {
        const uint8_t* krow = kt + t * C::KPITCH;
#pragma unroll 2
        for (int c = 0; c < C::PPR; ++c) {   // 4 dims per 16-B piece
          const float4 kx = *reinterpret_cast<const float4*>(krow + 16 * c);
#pragma unroll
          for (int j = 0; j < NH; ++j) {
            const float4 q4 = *reinterpret_cast<const float4*>(q_s + (hs + C::NHS * j) * C::QW + 4 * c);
            float a = dot[j];
            a = __builtin_fmaf(q4.x, kx.x, a);
            a = __builtin_fmaf(q4.y, kx.y, a);
            a = __builtin_fmaf(q4.z, kx.z, a);
            a = __builtin_fmaf(q4.w, kx.w, a);
            dot[j] = a;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const int g = hs + C::NHS * j;
        if (g < G) sc[g * T + t] = t < nc ? dot[j] * p.scale_log2 : -INFINITY;
      }
    }
    __syncthreads();
    // -------- online softmax: wave w takes heads w, w + 8
    for (int g = wave; g < G; g += kWinThreads / 64) {
      constexpr int R = T / 64;
      float x[R];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        x[r] = sc[g * T + lane + 64 * r];
        mx = fmaxf(mx, x[r]);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_old = s_m[g];
      const float m_new = fmaxf(m_old, mx);   // finite: the chunk holds at least one token
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float e = __builtin_amdgcn_exp2f(x[r] - m_new);   // -inf -> 0
        sc[g * T + lane + 64 * r] = e;
        sum += e;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      if (lane == 0) {
        const float alpha = m_old == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_old - m_new);
        s_a[g] = alpha;
        s_l[g] = s_l[g] * alpha + sum;
        s_m[g] = m_new;
      }
    }
    __syncthreads();
    // -------- P.V: dims 2 dp, 2 dp + 1 of every head over token range ts
    {
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        const float alpha = s_a[g];
        acc[g][0] *= alpha;
        acc[g][1] *= alpha;
      }
      const int span = (((nc + C::NTS - 1) / C::NTS) + 3) & ~3;   // multiple of 4: aligned p reads
      const int t0 = ts * span;
      const int t1 = (t0 + span) < nc ? (t0 + span) : nc;
      for (int t = t0; t < t1; t += 4) {
        float2 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          // the last group of a range may reach up to 3 rows past it (still
          // inside the chunk's LDS rows); those rows, which may never have
          // been written, are replaced by zeros and get p = 0 below
          v[u] = *reinterpret_cast<const float2*>(vt + (t + u) * C::ROWB + 8 * dp);
          if (t + u >= t1) v[u] = float2{0.f, 0.f};
        }
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
          float4 pr = *reinterpret_cast<const float4*>(sc + g * T + t);
          pr.y = t + 1 < t1 ? pr.y : 0.f;   // (the last group of a range)
          pr.z = t + 2 < t1 ? pr.z : 0.f;
          pr.w = t + 3 < t1 ? pr.w : 0.f;
          float a0 = acc[g][0], a1 = acc[g][1];
          a0 = __builtin_fmaf(pr.x, v[0].x, a0); a1 = __builtin_fmaf(pr.x, v[0].y, a1);
          a0 = __builtin_fmaf(pr.y, v[1].x, a0); a1 = __builtin_fmaf(pr.y, v[1].y, a1);
          a0 = __builtin_fmaf(pr.z, v[2].x, a0); a1 = __builtin_fmaf(pr.z, v[2].y, a1);
          a0 = __builtin_fmaf(pr.w, v[3].x, a0); a1 = __builtin_fmaf(pr.w, v[3].y, a1);
          acc[g][0] = a0;
          acc[g][1] = a1;
        }
      }
    }
  }

  // -------- add the token ranges (LDS, over the K rows), normalise, merge
  // with the history partial, store
  __syncthreads();
  float* red = reinterpret_cast<float*>(kvt);   // [ts][g][D]
  static_assert(C::NTS * GMAX * D * 4 <= T * (C::KPITCH + C::ROWB), "range sums exceed the K/V row area");
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
    if (g < G) *reinterpret_cast<float2*>(red + (ts * G + g) * D + 2 * dp) = float2{acc[g][0], acc[g][1]};
  __syncthreads();
  for (int i = tid; i < G * (D / 2); i += kWinThreads) {
    const int g = i / (D / 2), d = 2 * (i % (D / 2));
    float o0 = 0.f, o1 = 0.f;
#pragma unroll 4
    for (int r = 0; r < C::NTS; ++r) {
      const float2 x = *reinterpret_cast<const float2*>(red + (r * G + g) * D + d);
      o0 += x.x;
      o1 += x.y;
    }
    const int h = h0 + g;
    const float l = s_l[g];
    // window partial: o_w = acc / l, lse_w = ln 2 * (m + log2 l); empty: -inf
    const float lse_w = l > 0.f ? 0.69314718055994531f * (s_m[g] + __log2f(l)) : -INFINITY;
    o0 = l > 0.f ? o0 / l : 0.f;
    o1 = l > 0.f ? o1 / l : 0.f;
    float lse_out = lse_w;
    const int64_t off = ((int64_t)s * p.Hq + h) * D + d;
    if (p.hist_o) {
      const float lh = s_hl[g];
      const float M = fmaxf(lh, lse_w);
      if (M == -INFINITY) {
        o0 = o1 = 0.f;
      } else {
        const float wh = lh == -INFINITY ? 0.f : expf(lh - M);
        const float ww = lse_w == -INFINITY ? 0.f : expf(lse_w - M);
        const float den = wh + ww;
        float h0v = 0.f, h1v = 0.f;
        if (wh > 0.f) {
          const float2 oh = *reinterpret_cast<const float2*>(p.hist_o + off);
          h0v = (wh / den) * oh.x;
          h1v = (wh / den) * oh.y;
        }
        o0 = h0v + (ww / den) * o0;
        o1 = h1v + (ww / den) * o1;
        lse_out = M + logf(den);
      }
    }
    if (p.out_f32) {
      *reinterpret_cast<float2*>(static_cast<float*>(p.out) + off) = float2{o0, o1};
    } else {
      const uint32_t w = (uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16);
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.out) + off) = w;
    }
    if (d == 0 && p.lse) p.lse[(int64_t)s * p.Hq + h] = lse_out;
  }
}

// ---------------------------------------------------------------- bf16 rows
// The same walk for bf16 window rows, with both contractions on the matrix
// cores (window_item.h), one (sequence, kv head) per workgroup: chunks of T
// = 256 tokens (128 for d = 128 with more than 8 q heads per kv head, to fit
// LDS).
template <int D, int GMAX>
__global__ __launch_bounds__(kWinThreads) void window_bf16_kernel(WindowParams p) {
  constexpr int T = (D == 128 && GMAX == 16) ? 128 : 256;
  using C = WinItemCfg<D, GMAX, kWinThreads, T>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::BYTES];
  window_items_bf16<D, GMAX, kWinThreads, T, 1>(p, WinSink{}, (int)blockIdx.x, (int)blockIdx.x + 1, lds,
                                             (int)threadIdx.x);
}

template <int D>
void launch_window_f32(const WindowParams& wp, int grid, hipStream_t st) {
  if (wp.G <= 4) hipLaunchKernelGGL((window_f32_kernel<D, 4>), dim3((unsigned)grid), dim3(kWinThreads), 0, st, wp);
  else if (wp.G <= 8) hipLaunchKernelGGL((window_f32_kernel<D, 8>), dim3((unsigned)grid), dim3(kWinThreads), 0, st, wp);
  else hipLaunchKernelGGL((window_f32_kernel<D, 16>), dim3((unsigned)grid), dim3(kWinThreads), 0, st, wp);
}

template <int D>
void launch_window_bf16(const WindowParams& wp, int grid, hipStream_t st) {
  if (wp.G <= 4) hipLaunchKernelGGL((window_bf16_kernel<D, 4>), dim3((unsigned)grid), dim3(kWinThreads), 0, st, wp);
  else if (wp.G <= 8) hipLaunchKernelGGL((window_bf16_kernel<D, 8>), dim3((unsigned)grid), dim3(kWinThreads), 0, st, wp);
  else hipLaunchKernelGGL((window_bf16_kernel<D, 16>), dim3((unsigned)grid), dim3(kWinThreads), 0, st, wp);
}

}  // namespace
}  // namespace tq

using namespace tq;

extern "C" tq_status tq_decode_dense(const void* q, tq_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, const void* k, const void* v,
                                     tq_dtype kv_dtype, int32_t capacity, const int32_t* lens, float scale,
                                     const float* hist_out, const float* hist_lse, void* out,
                                     tq_dtype out_dtype, float* lse, int32_t* dev_err, tq_stream_t stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || capacity < 0)
    return set_error(TQ_ERR_VALUE, "bad window shape");
  if (num_q_heads % num_kv_heads != 0) return set_error(TQ_ERR_VALUE, "num_q_heads must be a multiple of num_kv_heads");
  if (num_q_heads / num_kv_heads > kWinMaxG)
    return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "more than 16 q heads per kv head");
  if (head_dim != 64 && head_dim != 128) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "head_dim must be 64 or 128");
  if ((q_dtype != TQ_BF16 && q_dtype != TQ_F32) || (kv_dtype != TQ_BF16 && kv_dtype != TQ_F32) ||
      (out_dtype != TQ_BF16 && out_dtype != TQ_F32))
    return set_error(TQ_ERR_VALUE, "dtypes must be BF16 or F32");
  if (!(scale > 0.f) || !std::isfinite(scale)) return set_error(TQ_ERR_VALUE, "scale must be finite and > 0");
  if ((hist_out == nullptr) != (hist_lse == nullptr))
    return set_error(TQ_ERR_VALUE, "hist_out and hist_lse go together");
  if ((int64_t)num_seqs * num_kv_heads >= (int64_t)1 << 31) return set_error(TQ_ERR_VALUE, "too many (sequence, kv head) pairs");
  if (num_seqs == 0) return TQ_OK;
  if (!q || !lens || !out) return set_error(TQ_ERR_VALUE, "NULL q, lens or out");
  if (capacity > 0 && (!k || !v)) return set_error(TQ_ERR_VALUE, "NULL window K or V");
  if (((uintptr_t)k | (uintptr_t)v) & 15u) return set_error(TQ_ERR_VALUE, "window K and V must be 16-byte aligned");
  if (((uintptr_t)q | (uintptr_t)out | (uintptr_t)hist_out) & 7u)
    return set_error(TQ_ERR_VALUE, "q, out and hist_out must be 8-byte aligned");
  WindowParams wp;
  wp.q = q; wp.k = k; wp.v = v; wp.lens = lens;
  wp.hist_o = hist_out; wp.hist_lse = hist_lse;
  wp.out = out; wp.lse = lse; wp.dev_err = dev_err;
  wp.S = num_seqs; wp.Hq = num_q_heads; wp.Hkv = num_kv_heads; wp.G = num_q_heads / num_kv_heads;
  wp.cap = capacity;
  wp.scale_log2 = (float)((double)scale * 1.4426950408889634);
  wp.q_f32 = q_dtype == TQ_F32;
  wp.out_f32 = out_dtype == TQ_F32;
  const int grid = num_seqs * num_kv_heads;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool kv32 = kv_dtype == TQ_F32;
  if (head_dim == 128) {
    if (kv32) launch_window_f32<128>(wp, grid, st);
    else launch_window_bf16<128>(wp, grid, st);
  } else {
    if (kv32) launch_window_f32<64>(wp, grid, st);
    else launch_window_bf16<64>(wp, grid, st);
  }
  return launch_status("tq_decode_dense launch");
}
