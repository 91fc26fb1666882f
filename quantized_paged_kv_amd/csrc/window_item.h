// Exact attention of the q heads of one (sequence, kv head) over a dense
// window of bf16 K / V rows, walked in chunks of T tokens by NT threads with
// both contractions on the matrix cores; the result goes to the output
// (optionally merged with a history partial by the log-sum-exp identity) or
// to one partial slot of the split merge.  Used by the dense-window kernel
// and, after the packed history, by the paged decode kernel.
//
// Per chunk of T tokens:
//   scores  wave w takes 16-token tiles w, w + NT/64: S = K Q^T by
//           v_mfma_f32_16x16x32_bf16 (A = 16 K rows x 32 dims straight from
//           the staged rows, B = 32 dims x 16 q heads); bf16 products are
//           exact and sums fp32 (an f32 q is instead multiplied in fp32 FMAs,
//           thread per token);
//   softmax wave w takes heads w, w + NT/64: max and sum by DPP/permlane
//           exchanges, p = 2^(s - m) split into a bf16 high part and the bf16
//           rounding of the rest (p_hi + p_lo = p to 2^-17), written as two
//           [head][token] planes;
//   P.V     wave w takes dims 16 w .. 16 w + 15 over all token tiles:
//           O^T += V^T P by v_mfma_f32_16x16x16_bf16, once with p_hi and once
//           with p_lo (A = 16 dims x 16 tokens gathered from the staged V
//           rows, B = 16 tokens x 16 q heads from the planes).
// The chunk's K and V rows are staged in LDS by coalesced 16-B loads, all
// issued before any is waited for (the next chunk's while this one is
// computed), so a chunk costs one memory round trip.
#pragma once

#include "tq_internal.h"

namespace tq {
namespace {

struct WindowParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* lens;
  const float* hist_o;     // [S][Hq][D] f32 or NULL
  const float* hist_lse;   // [S][Hq] or NULL
  void* out;
  float* lse;
  int32_t* dev_err;
  int32_t S, Hq, Hkv, G, cap;
  float scale_log2;   // softmax scale times log2(e): scores live in the base-2 domain
  int32_t q_f32, out_f32;
};

// Where a window item's result goes: part_o == NULL: the output (merged with
// the history partial if given); else slot `slot` of rows of PS partial
// slots, normalised output and natural-log lse (-inf for an empty window).
struct WinSink {
  float* part_o = nullptr;
  float* part_lse = nullptr;
  int PS = 0, slot = 0;
};

// LDS layout of a window item (byte offsets from its base).
template <int D, int GMAX, int NT, int TT>
struct WinItemCfg {
  static constexpr int T = TT;              // tokens per chunk
  static constexpr int ROWB = D * 2;
  static constexpr int PITCH = ROWB + 16;   // staged K and V rows: rows 4 apart sit 16 banks apart
  static constexpr int PPR = ROWB / 16;     // 16-B pieces per row
  static constexpr int NPC = T * PPR / NT;  // pieces per thread per tensor
  static constexpr int TP = T + 4;          // p planes: u16 per head row (8-B aligned reads)
  static constexpr int QW = D + 4;          // q row in LDS (words)
  static constexpr int NHS = NT / T;        // head sets of the fp32 score path
  static_assert(NPC * NT == T * PPR && NHS * T == NT && T % 64 == 0, "window chunk does not fit the threads");
  static constexpr int PLANE = (GMAX * TP * 2 + 15) / 16 * 16;
  static constexpr int OFF_KT = 0;
  static constexpr int OFF_VT = OFF_KT + T * PITCH;
  static constexpr int OFF_SC = OFF_VT + T * PITCH;
  static constexpr int OFF_PHI = OFF_SC + GMAX * T * 4;
  static constexpr int OFF_PLO = OFF_PHI + PLANE;
  static constexpr int OFF_Q = OFF_PLO + PLANE;
  static constexpr int OFF_ML = OFF_Q + GMAX * QW * 4;
  static constexpr int BYTES = OFF_ML + 4 * GMAX * 4;
};

typedef __bf16 win_bf16x8 __attribute__((ext_vector_type(8)));
typedef short win_s16x4 __attribute__((ext_vector_type(4)));
typedef float win_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t win_u32x4 __attribute__((ext_vector_type(4)));   // 16-B row piece (a plain vector value)

// Rows of one chunk in flight: thread tid holds 16-B pieces tid + NT i
// (row (tid + NT i) / PPR, piece (tid + NT i) % PPR) of K and of V.
template <int NPC>
struct WinRows {
  win_u32x4 k[NPC], v[NPC];
};

// Requests rows c0 .. c0 + T - 1 (those below lim) of the window rows at
// byte offset base.
template <int D, int GMAX, int NT, int TT>
__device__ __forceinline__ void win_issue_rows(WinRows<WinItemCfg<D, GMAX, NT, TT>::NPC>& r, const WindowParams& p,
                                               int64_t base, int c0, int lim, int tid) {
  using C = WinItemCfg<D, GMAX, NT, TT>;
  const int64_t row_bytes = (int64_t)p.Hkv * C::ROWB;
#pragma unroll
  for (int i = 0; i < C::NPC; ++i) {
    const int pc = tid + NT * i;
    const int t = pc / C::PPR, c = pc % C::PPR;
    const int64_t off = base + (int64_t)(c0 + t) * row_bytes + 16 * c;
    if (c0 + t < lim) {
      r.k[i] = *reinterpret_cast<const win_u32x4*>(static_cast<const uint8_t*>(p.k) + off);
      r.v[i] = *reinterpret_cast<const win_u32x4*>(static_cast<const uint8_t*>(p.v) + off);
    }
  }
}

// Byte offset of row 0 of item it (= s * Hkv + kv head).
template <int D>
__device__ __forceinline__ int64_t win_item_base(const WindowParams& p, int it) {
  return ((int64_t)(it / p.Hkv) * p.cap * p.Hkv + it % p.Hkv) * (2 * D);
}

// Requests item it's q pairs, its window length and its first DEPTH chunks
// (speculatively: the length is not known yet, so up to the capacity).
template <int D, int GMAX, int NT, int TT, int DEPTH, int QPT>
__device__ __forceinline__ void win_issue_item(WinRows<WinItemCfg<D, GMAX, NT, TT>::NPC>& r0,
                                               WinRows<WinItemCfg<D, GMAX, NT, TT>::NPC>& r1, uint2 (&qv)[QPT],
                                               int& n_next, const WindowParams& p, int it, int tid) {
  const int s = it / p.Hkv, h0 = (it % p.Hkv) * p.G;
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int i = tid + NT * j;
    if (i < p.G * (D / 2)) {
      const int64_t off = ((int64_t)s * p.Hq + h0) * D + 2 * i;
      if (p.q_f32) qv[j] = *reinterpret_cast<const uint2*>(static_cast<const float*>(p.q) + off);
      else qv[j].x = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.q) + off);
    }
  }
  n_next = p.lens[s];
  const int64_t base = win_item_base<D>(p, it);
  const int lim = p.cap < DEPTH * TT ? p.cap : DEPTH * TT;
  win_issue_rows<D, GMAX, NT, TT>(r0, p, base, 0, lim, tid);
  if constexpr (DEPTH == 2) win_issue_rows<D, GMAX, NT, TT>(r1, p, base, TT, lim, tid);
}

// Stages chunk c0 (n tokens in all) into LDS.  V rows past the chunk's
// tokens (up to the tile boundary) are zeros: they meet p = 0 in the
// products.
template <int D, int GMAX, int NT, int TT>
__device__ __forceinline__ void win_stage(const WinRows<WinItemCfg<D, GMAX, NT, TT>::NPC>& r, uint8_t* lds, int c0,
                                          int n, int tid) {
  using C = WinItemCfg<D, GMAX, NT, TT>;
  const int nc = (n - c0) < TT ? (n - c0) : TT;
  const int ntt = (nc + 15) >> 4;
  if (c0 > 0) __syncthreads();   // the previous chunk's rows and planes have been read
#pragma unroll
  for (int i = 0; i < C::NPC; ++i) {
    const int pc = tid + NT * i;
    const int t = pc / C::PPR, c = pc % C::PPR;
    if (t < nc) *reinterpret_cast<win_u32x4*>(lds + C::OFF_KT + t * C::PITCH + 16 * c) = r.k[i];
    if (t < 16 * ntt)
      *reinterpret_cast<win_u32x4*>(lds + C::OFF_VT + t * C::PITCH + 16 * c) = t < nc ? r.v[i] : win_u32x4{0u, 0u, 0u, 0u};
  }
}

// Scores, online softmax and P.V of the staged chunk c0 (n tokens in all);
// acc is this lane's P.V cell O^T[16 wave + 4 grp + i][col].
template <int D, int GMAX, int NT, int TT>
__device__ __forceinline__ void win_compute(const WindowParams& p, uint8_t* lds, int c0, int n, int tid,
                                            win_f32x4& acc) {
  using C = WinItemCfg<D, GMAX, NT, TT>;
  constexpr int T = TT;
  constexpr int NDT = D / 16;
  const uint8_t* const kt = lds + C::OFF_KT;
  const uint8_t* const vt = lds + C::OFF_VT;
  float* const sc = reinterpret_cast<float*>(lds + C::OFF_SC);
  uint16_t* const phi = reinterpret_cast<uint16_t*>(lds + C::OFF_PHI);
  uint16_t* const plo = reinterpret_cast<uint16_t*>(lds + C::OFF_PLO);
  const uint32_t* const q_s = reinterpret_cast<const uint32_t*>(lds + C::OFF_Q);
  float* const s_m = reinterpret_cast<float*>(lds + C::OFF_ML);
  float* const s_l = s_m + GMAX;
  float* const s_a = s_m + 2 * GMAX;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  const int col = lane & 15, grp = lane >> 4;
  const int gl = col < GMAX ? col : GMAX - 1;
  const int nc = (n - c0) < T ? (n - c0) : T;
  const int ntt = (nc + 15) >> 4;   // 16-token tiles
  __syncthreads();
  // -------- scores (base-2 domain)
  if (!p.q_f32) {
    for (int tt = wave; tt < ntt; tt += NT / 64) {
      win_f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = kt + (16 * tt + col) * C::PITCH + 16 * grp;
      const uint32_t* qrow = q_s + gl * C::QW + 4 * grp;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(krow + 64 * ks);
        const uint4 b = *reinterpret_cast<const uint4*>(qrow + 16 * ks);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(win_bf16x8, a),
                                                       __builtin_bit_cast(win_bf16x8, b), sacc, 0, 0, 0);
      }
      if (col < G) {   // rows 4 grp + i of the tile: tokens; column: q head
        const int t = 16 * tt + 4 * grp;
        float4 o;
        o.x = t < nc ? sacc[0] * p.scale_log2 : -INFINITY;
        o.y = t + 1 < nc ? sacc[1] * p.scale_log2 : -INFINITY;
        o.z = t + 2 < nc ? sacc[2] * p.scale_log2 : -INFINITY;
        o.w = t + 3 < nc ? sacc[3] * p.scale_log2 : -INFINITY;
        *reinterpret_cast<float4*>(sc + col * T + t) = o;
      }
    }
  } else {   // f32 q: fp32 FMAs, thread per token of the chunk, heads hs, hs + NHS, ...
    const int t = tid % T;
    const int hs = __builtin_amdgcn_readfirstlane(tid / T);
    constexpr int NH = (GMAX + C::NHS - 1) / C::NHS;
    float dot[NH];
#pragma unroll
    for (int j = 0; j < NH; ++j) dot[j] = 0.f;
    if (t < nc) {
      const uint8_t* krow = kt + t * C::PITCH;
#pragma unroll 2
      for (int c = 0; c < C::PPR; ++c) {
        const uint4 kw = *reinterpret_cast<const uint4*>(krow + 16 * c);
        const uint32_t u[4] = {kw.x, kw.y, kw.z, kw.w};
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = __uint_as_float(u[e] << 16);
          x[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
        }
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          const int g = hs + C::NHS * j;
          const float* qf = reinterpret_cast<const float*>(q_s + (g < GMAX ? g : GMAX - 1) * C::QW) + 8 * c;
          const float4 q0 = *reinterpret_cast<const float4*>(qf);
          const float4 q1 = *reinterpret_cast<const float4*>(qf + 4);
          float a = dot[j];
          a = __builtin_fmaf(q0.x, x[0], a); a = __builtin_fmaf(q0.y, x[1], a);
          a = __builtin_fmaf(q0.z, x[2], a); a = __builtin_fmaf(q0.w, x[3], a);
          a = __builtin_fmaf(q1.x, x[4], a); a = __builtin_fmaf(q1.y, x[5], a);
          a = __builtin_fmaf(q1.z, x[6], a); a = __builtin_fmaf(q1.w, x[7], a);
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
  // -------- online softmax: wave w takes heads w, w + NT / 64; tokens past
  // the chunk count as -inf (their plane entries become 0)
  for (int g = wave; g < G; g += NT / 64) {
    constexpr int R = T / 64;
    float x[R];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int t = lane + 64 * r;
      x[r] = t < nc ? sc[g * T + t] : -INFINITY;
      mx = fmaxf(mx, x[r]);
    }
    mx = fmaxf(mx, lane_xor<32>(mx, lane));
    mx = fmaxf(mx, lane_xor<16>(mx, lane));
    mx = fmaxf(mx, lane_xor<8>(mx, lane));
    mx = fmaxf(mx, lane_xor<4>(mx, lane));
    mx = fmaxf(mx, lane_xor<2>(mx, lane));
    mx = fmaxf(mx, lane_xor<1>(mx, lane));
    const float m_old = s_m[g];
    const float m_new = fmaxf(m_old, mx);   // finite: the chunk holds at least one token
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float e = __builtin_amdgcn_exp2f(x[r] - m_new);   // -inf -> 0
      sum += e;
      const uint16_t hi = f32_to_bf16_rne(e);
      const float rest = e - __uint_as_float((uint32_t)hi << 16);
      phi[g * C::TP + lane + 64 * r] = hi;
      plo[g * C::TP + lane + 64 * r] = f32_to_bf16_rne(rest);
    }
    sum += lane_xor<32>(sum, lane);
    sum += lane_xor<16>(sum, lane);
    sum += lane_xor<8>(sum, lane);
    sum += lane_xor<4>(sum, lane);
    sum += lane_xor<2>(sum, lane);
    sum += lane_xor<1>(sum, lane);
    if (lane == 0) {
      const float alpha = m_old == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_old - m_new);
      s_a[g] = alpha;
      s_l[g] = s_l[g] * alpha + sum;
      s_m[g] = m_new;
    }
  }
  __syncthreads();
  // -------- P.V: wave w, dims 16 w .. 16 w + 15
  if (wave < NDT) {
    const float alpha = s_a[gl];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= alpha;
    const uint8_t* vcol = vt + 2 * (16 * wave + col) + (4 * grp) * C::PITCH;   // dim 16 w + col, token 4 grp
    const uint16_t* ph = phi + gl * C::TP + 4 * grp;
    const uint16_t* pl = plo + gl * C::TP + 4 * grp;
    for (int tt = 0; tt < ntt; ++tt) {
      const uint8_t* v0 = vcol + (16 * tt) * C::PITCH;
      const uint32_t a0 = *reinterpret_cast<const uint16_t*>(v0);
      const uint32_t a1 = *reinterpret_cast<const uint16_t*>(v0 + C::PITCH);
      const uint32_t a2 = *reinterpret_cast<const uint16_t*>(v0 + 2 * C::PITCH);
      const uint32_t a3 = *reinterpret_cast<const uint16_t*>(v0 + 3 * C::PITCH);
      const uint2 av = uint2{a0 | (a1 << 16), a2 | (a3 << 16)};   // V[t0 + 4 grp + i][dim], i = 0..3
      const uint2 bh = *reinterpret_cast<const uint2*>(ph + 16 * tt);
      const uint2 bl = *reinterpret_cast<const uint2*>(pl + 16 * tt);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(win_s16x4, av),
                                                      __builtin_bit_cast(win_s16x4, bh), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(win_s16x4, av),
                                                      __builtin_bit_cast(win_s16x4, bl), acc, 0, 0, 0);
    }
  }
}

// Items it0 .. it1 - 1 (item = s * Hkv + kv head) one after another, with
// DEPTH (1 or 2) chunks of rows in flight: chunk c + DEPTH is requested as
// chunk c is staged, and the loads of an item (its q rows, window length
// and first DEPTH chunks) during the last chunk of the item before, so a
// run of items costs no extra memory round trip per item, and with DEPTH 2
// two chunks share one.
template <int D, int GMAX, int NT, int TT, int DEPTH>
__device__ __forceinline__ void window_items_bf16(const WindowParams& p, const WinSink& sink, int it0, int it1,
                                                  uint8_t* lds, int tid) {
  using C = WinItemCfg<D, GMAX, NT, TT>;
  constexpr int T = C::T;
  constexpr int NDT = D / 16;   // 16-dim tiles (one per wave in P.V)
  static_assert(DEPTH == 1 || DEPTH == 2, "one or two chunks in flight");
  uint32_t* const q_s = reinterpret_cast<uint32_t*>(lds + C::OFF_Q);     // bf16 pairs, or f32 (f32 q)
  float* const s_m = reinterpret_cast<float*>(lds + C::OFF_ML);
  float* const s_l = s_m + GMAX;
  float* const s_hl = s_m + 3 * GMAX;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  const int col = lane & 15, grp = lane >> 4;   // MFMA lane coordinates
  constexpr int QPT = (GMAX * D / 2 + NT - 1) / NT;

  // in flight: q pairs and the window length of the next item, and the
  // rows of DEPTH chunks (r0: chunks c with c % DEPTH == 0, r1: the others)
  uint2 qv[QPT];
  WinRows<C::NPC> r0, r1;
  int n_next = 0;
  if (it0 >= it1) return;
  win_issue_item<D, GMAX, NT, TT, DEPTH, QPT>(r0, r1, qv, n_next, p, it0, tid);
  for (int it = it0; it < it1; ++it) {
    const int s = it / p.Hkv, kvh = it % p.Hkv;
    const int h0 = kvh * G;
    const int64_t base = win_item_base<D>(p, it);
    const bool more = it + 1 < it1;
    // history partial (the output path): lse and this lane's output cell,
    // head col, dims 16 wave + 4 grp .. + 3
    const float hl_own = (tid < G && p.hist_lse) ? p.hist_lse[(int64_t)s * p.Hq + h0 + tid] : -INFINITY;
    const int64_t out_off = ((int64_t)s * p.Hq + h0 + col) * D + 16 * wave + 4 * grp;
    float4 hv = float4{0.f, 0.f, 0.f, 0.f};
    if (p.hist_o && wave < NDT && col < G) hv = *reinterpret_cast<const float4*>(p.hist_o + out_off);
    int n = n_next;
    if (n < 0 || n > p.cap) {
      if (tid == 0 && kvh == 0) record_error(p.dev_err, TQ_ERR_INDEX, -1 - s);
      n = n < 0 ? 0 : p.cap;
    }
    __syncthreads();   // the item before is done with q, the running values and the planes
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int i = tid + NT * j;
      if (i < G * (D / 2)) {
        const int g = i / (D / 2), dp = i % (D / 2);
        if (!p.q_f32) {
          q_s[g * C::QW + dp] = qv[j].x;
        } else {
          q_s[g * C::QW + 2 * dp] = qv[j].x;
          q_s[g * C::QW + 2 * dp + 1] = qv[j].y;
        }
      }
    }
    if (tid < G) {
      s_m[tid] = -INFINITY;
      s_l[tid] = 0.f;
      s_hl[tid] = hl_own;
    }
    if (n == 0 && more) win_issue_item<D, GMAX, NT, TT, DEPTH, QPT>(r0, r1, qv, n_next, p, it + 1, tid);

    win_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < n; c0 += DEPTH * T) {
      // each buffer, once staged, takes chunk c + DEPTH, or after the item's
      // last chunk the next item's loads: their round trip overlaps the
      // arithmetic
      win_stage<D, GMAX, NT, TT>(r0, lds, c0, n, tid);
      if (c0 + DEPTH * T < n) win_issue_rows<D, GMAX, NT, TT>(r0, p, base, c0 + DEPTH * T, n, tid);
      else if (c0 + T >= n && more) win_issue_item<D, GMAX, NT, TT, DEPTH, QPT>(r0, r1, qv, n_next, p, it + 1, tid);
      win_compute<D, GMAX, NT, TT>(p, lds, c0, n, tid, acc);
      if constexpr (DEPTH == 2) {
        const int c1 = c0 + T;
        if (c1 < n) {
          win_stage<D, GMAX, NT, TT>(r1, lds, c1, n, tid);
          if (c1 + DEPTH * T < n) win_issue_rows<D, GMAX, NT, TT>(r1, p, base, c1 + DEPTH * T, n, tid);
          else if (c1 + T >= n && more) win_issue_item<D, GMAX, NT, TT, DEPTH, QPT>(r0, r1, qv, n_next, p, it + 1, tid);
          win_compute<D, GMAX, NT, TT>(p, lds, c1, n, tid, acc);
        }
      }
    }
    __syncthreads();   // s_l / s_m of the last chunk (and an empty window's initial values)

    // -------- normalise, then store as a partial slot, or merged with the
    // history partial as the output: lane holds head col, dims 16 w + 4 grp .. + 3
    if (wave < NDT && col < G) {
      const float l = s_l[col];
      const float lse_w = l > 0.f ? 0.69314718055994531f * (s_m[col] + __log2f(l)) : -INFINITY;
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = l > 0.f ? acc[i] / l : 0.f;
      if (sink.part_o) {   // one partial slot of the split merge
        const int64_t row = ((int64_t)s * p.Hq + h0 + col) * sink.PS + sink.slot;
        *reinterpret_cast<float4*>(sink.part_o + row * D + 16 * wave + 4 * grp) = float4{o[0], o[1], o[2], o[3]};
        if (wave == 0 && grp == 0) sink.part_lse[row] = lse_w;
      } else {
        float lse_out = lse_w;
        if (p.hist_o) {
          const float lh = s_hl[col];
          const float M = fmaxf(lh, lse_w);
          if (M == -INFINITY) {
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = 0.f;
          } else {
            const float wh = lh == -INFINITY ? 0.f : expf(lh - M);
            const float ww = lse_w == -INFINITY ? 0.f : expf(lse_w - M);
            const float den = wh + ww;
            const float ah = wh / den, aw = ww / den;
            const float h[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (wh > 0.f ? ah * h[i] : 0.f) + aw * o[i];
            lse_out = M + logf(den);
          }
        }
        if (p.out_f32) {
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + out_off) = float4{o[0], o[1], o[2], o[3]};
        } else {
          const uint2 w = uint2{(uint32_t)f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16),
                                (uint32_t)f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16)};
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + out_off) = w;
        }
        if (wave == 0 && grp == 0 && p.lse) p.lse[(int64_t)s * p.Hq + h0 + col] = lse_out;
      }
    }
  }
}


}  // namespace
}  // namespace tq
