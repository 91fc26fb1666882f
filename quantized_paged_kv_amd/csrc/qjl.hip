// QJL residual stage of K channel groups: the write-side kernel that adds
// each row's sign sketch and residual norm, and the decode kernel that adds
// the sketch's estimate to every score.
//
// [D "Recipe Strategy"]: each group of a recipe row stores [MSE indices]
// [QJL signs][vector norm][residual norm].  The pages give the fields, not
// the stage; the one implemented is the quantised Johnson-Lindenstrauss
// transform as published with TurboQuant's inner-product quantiser: the
// group's MSE residual r is projected by a caller-supplied m x m Gaussian
// matrix S, the signs of S r are stored with |r|, and a query q adds
// sqrt(pi/2) / m * |r| * <S q, signs> to its score (unbiased for <q, r>).
//
// Write side (fp64, no fused multiply-add anywhere): the
// rotation is recomputed with the same butterflies as the MSE stage, the
// stored indices and norm are read back from the tile the MSE kernel wrote
// just before on the same stream, and
//   r_j = w_j - (norm * sqrt(d/m)) * c[idx_j],  rnorm = fp16(sqrt(tree(r^2) / d)),
//   bit_i = (sum_j S[i][j] r_j < 0), the sum taken from +0 over j ascending,
//           each product and each partial sum rounded to fp64 in turn.
//
// Decode: one 8-wave workgroup per (sequence, kv head, split).  Every wave
// takes every 8th block of the split, stages the K and V tiles in LDS and
// runs the scores on the matrix cores as one contraction over 2d "channels":
// [rotated q | projected q] (fp16 high + low parts, columns 0-7 / 8-15)
// against [codebook values | +-rnorm] of the 16 tokens (both exact in fp16),
// one fp32 accumulator per MSE group and one for the sketch; softmax in the
// exp2 domain; P.V on the matrix cores with the V codebook values.  The
// waves' states are combined in LDS, the result is rotated back and written
// out, or as a partial for the split merge.
#pragma clang fp contract(off)

#include <math.h>

#include <algorithm>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void wave_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

__device__ __forceinline__ int norm_slot(int t) { return 4 * (t & 3) + (t >> 2); }

// ------------------------------------------------------------------ write

constexpr int kWriteWaves = 4;
constexpr int kProjMax = 128 * 129;   // padded projection floats (one group of 128, or two of 64)

struct QjlWriteParams {
  QjlWriteArgs a;
  DevFormat f;
};

// fp64 sum over the lanes of aligned groups of `span` lanes (span a power of
// two <= 64) by the pairwise tree: level o adds lane l ^ o, which is the
// adjacent-pairs-first order of the group's elements.
__device__ __forceinline__ double group_tree_sum(double v, int span, int lane) {
  if (span > 1) v += lane_xor_d<1>(v, lane);
  if (span > 2) v += lane_xor_d<2>(v, lane);
  if (span > 4) v += lane_xor_d<4>(v, lane);
  if (span > 8) v += lane_xor_d<8>(v, lane);
  if (span > 16) v += lane_xor_d<16>(v, lane);
  if (span > 32) v += lane_xor_d<32>(v, lane);
  return v;
}

template <int D, bool F32>
__global__ __launch_bounds__(64 * kWriteWaves) void qjl_write_kernel(QjlWriteParams p) {
  constexpr int KP = D / 64;   // positions (and projection outputs) per lane
  __shared__ float sproj[kProjMax];
  __shared__ double sw[kWriteWaves][D];
  __shared__ double sr[kWriteWaves][D];
  const DevFormat& f = p.f;
  const int m = f.m, ng = f.ng;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // projection rows padded to m + 1 floats (lanes read different rows);
  // every 16-byte load of a thread is issued before any is stored, so the
  // staging costs one memory round trip (ng m m = D m <= 16384 floats:
  // at most 16 loads per thread)
  {
    constexpr int NV = D * D / 4 / (64 * kWriteWaves);   // float4 per thread when m = D (the most)
    float4 v[NV];
    const int n4 = ng * m * m / 4;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int e = tid + 64 * kWriteWaves * k;
      if (e < n4) v[k] = reinterpret_cast<const float4*>(p.a.proj)[e];
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int e = tid + 64 * kWriteWaves * k;
      if (e < n4) {
        const int row = (4 * e) / m, j = 4 * e - row * m;
        float* dst = sproj + row * (m + 1) + j;
        dst[0] = v[k].x; dst[1] = v[k].y; dst[2] = v[k].z; dst[3] = v[k].w;
      }
    }
  }
  __syncthreads();
  const int64_t rows = p.a.num_tokens * p.a.H;
  double* w = sw[wave];
  double* r = sr[wave];
  for (int64_t row = (int64_t)blockIdx.x * kWriteWaves + wave; row < rows;
       row += (int64_t)gridDim.x * kWriteWaves) {
    const int64_t tok = row / p.a.H;
    const int h = (int)(row - tok * p.a.H);
    const int64_t slot = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)p.a.slots[tok]) |
                         ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)p.a.slots[tok] >> 32)) << 32);
    if (slot < 0 || slot >= p.a.num_slots) continue;   // reported by the MSE write (wave-uniform)
    uint8_t* tile = p.a.pages + ((slot >> 4) * p.a.H + h) * (int64_t)f.tile_bytes;
    const int offs = (int)(slot & 15);
    const uint8_t* rowb = tile + offs * f.row_bytes;
    // signs, then the butterflies h = 1, 2, ..., D/2 in fp64
    for (int c = lane; c < D; c += 64) {
      double x;
      if constexpr (F32) x = (double)static_cast<const float*>(p.a.src)[row * D + c];
      else x = (double)__uint_as_float((uint32_t)static_cast<const uint16_t*>(p.a.src)[row * D + c] << 16);
      if ((f.sign_bits[c >> 5] >> (c & 31)) & 1u) x = -x;
      w[c] = x;
    }
    for (int hs = 1; hs < D; hs <<= 1) {
      wave_fence();
      for (int pr = lane; pr < D / 2; pr += 64) {
        const int i = (pr / hs) * 2 * hs + (pr % hs), j = i + hs;
        const double a0 = w[i], b0 = w[j];
        w[i] = a0 + b0;
        w[j] = a0 - b0;
      }
    }
    wave_fence();
    // residual at group position P = lane + 64 k (group P / m, position P % m)
    double rv[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int P = lane + 64 * k;
      const int g = P / m, pos = P - g * m;
      const int bits = f.bits[g];
      const int bit0 = pos * bits;
      const int byte = f.grp_byte_off[g] + (bit0 >> 3);
      const uint32_t two = (uint32_t)rowb[byte] | ((uint32_t)rowb[byte + 1] << 8);
      const int code = (int)((two >> (bit0 & 7)) & ((1u << bits) - 1u));
      const uint16_t nb = *reinterpret_cast<const uint16_t*>(tile + f.norm_off + 2 * (16 * g + norm_slot(offs)));
      const double a = f16_bits_to_f64(nb) * p.a.kappa;
      const double t = a * f16_bits_to_f64(f.cb[g][code]);
      rv[k] = w[f.ch[P]] - t;
      r[P] = rv[k];
    }
    // residual norm per group: pairwise tree over the group's positions
    double ss[2] = {0.0, 0.0};
    if (m >= 64) {
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const double v = group_tree_sum(rv[k] * rv[k], 64, lane);
        const int g = (64 * k) / m;
        ss[g] = (64 * k) % m == 0 ? v : ss[g] + v;   // m = 128: (0..63) + (64..127), the tree's last level
      }
    } else {   // m = 32 (D = 64, two groups): lanes 0-31 group 0, 32-63 group 1
      const double v = group_tree_sum(rv[0] * rv[0], 32, lane);
      ss[0] = __shfl(v, 0);
      ss[1] = __shfl(v, 32);
    }
    wave_fence();
    // projection z_i = sum_j S[i][j] r_j: from +0, j ascending, the product
    // and then the sum rounded to fp64 at every step (the file is compiled
    // without contraction, so the two operations stay separate); signs by
    // ballot
    uint64_t neg[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int O = lane + 64 * k;
      const int g = O / m, i = O - g * m;
      const float* srow = sproj + (g * m + i) * (m + 1);
      const double* rg = r + g * m;
      double z = 0.0;
      for (int j = 0; j < m; ++j) z = z + (double)srow[j] * rg[j];
      neg[k] = __builtin_amdgcn_ballot_w64(z < 0.0);
    }
    uint8_t* sgn = tile + offs * f.row_bytes + f.sign_off;
#pragma unroll
    for (int k = 0; k < KP; ++k)
      if (lane < 8) sgn[8 * k + lane] = (uint8_t)(neg[k] >> (8 * lane));
    if (lane < ng) {
      const double s = lane == 0 ? ss[0] : ss[1];
      *reinterpret_cast<uint16_t*>(tile + f.rnorm_off + 2 * (16 * lane + norm_slot(offs))) =
          f64_to_f16_rne(__builtin_sqrt(s / (double)D));
    }
  }
}

// ------------------------------------------------------------------ decode

constexpr int kDecWaves = 8;
constexpr int kKTileMax = 1536;
constexpr int kVTileMax = 1088;

struct QjlDecParams {
  QjlDecodeArgs a;
  DevFormat kf, vf;
  float f_mse, f_q;   // score factors (log2 units): scale log2e / sqrt(m d), scale log2e sqrt(pi/2) / (m sqrt d)
};

template <int D, int NG, int VB>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(4))) void qjl_decode_kernel(QjlDecParams p) {
  constexpr int M = D / NG;         // channels per K group
  constexpr int VC = D / 16 * VB / 8;   // V bytes per token in one lane's run of the lane-major plane
  constexpr int NT = D / 32;        // MSE contractions of 32 channels (and as many sketch ones)
  constexpr int ND = D / 16;        // P.V contractions of 16 dims
  __shared__ float qg[8][D];        // rotated query (unnormalised), then in group position order
  __shared__ float qt[8][D];        // scratch: rotation, then the projected query
  __shared__ half8_t bop[2 * NT][64];
  __shared__ float wmse[8], wq[8];
  __shared__ uint16_t cbv[16];
  __shared__ uint32_t vpair[16];         // 2-bit V: two codes (c0 | c1 << 2) -> (cb[c0], cb[c1])
  __shared__ uint32_t cbpair[NG][256];   // per K group: two codes (c0 | c1 << bits) -> (cb[c0], cb[c1])
  __shared__ __attribute__((aligned(16))) uint8_t ktile[kDecWaves][kKTileMax];
  __shared__ __attribute__((aligned(16))) uint8_t vtile[kDecWaves][kVTileMax];
  __shared__ float st_o[kDecWaves][8][D];
  __shared__ float st_ml[kDecWaves][2][8];

  const QjlDecodeArgs& a = p.a;
  const DevFormat& kf = p.kf;
  const DevFormat& vf = p.vf;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.P;
  const int sp = blockIdx.x % P;
  const int rest = blockIdx.x / P;
  const int kvh = rest % a.Hkv;
  const int s = rest / a.Hkv;
  const int G = a.G;
  const int cap = a.max_blocks * 16;
  const int ctx_raw = a.context_lens[s];
  if (sp == 0 && kvh == 0 && tid == 0 && (ctx_raw < 0 || ctx_raw > cap)) record_error(a.dev_err, TQ_ERR_INDEX, -1 - s);
  const int ctx = ctx_raw < 0 ? 0 : (ctx_raw > cap ? cap : ctx_raw);
  const int nb = (ctx + 15) >> 4;
  const int cb = (nb + P - 1) / P;
  const int b0 = sp * cb;
  const int b1 = std::min(nb, b0 + cb);

  // Each wave keeps its next block's tiles in flight in registers (16 B at
  // 16 lane and 16 lane + 1024 of each) while it computes the current one
  // from LDS.  An entry outside the pool is reported when it is read and the
  // block is skipped (block 0 is loaded in its place, never used).
  auto entry_of = [&](int b, bool& ok) -> int {
    const int raw = __builtin_amdgcn_readfirstlane(a.block_tables[(int64_t)s * a.max_blocks + b]);
    ok = !(raw < 0 || (int64_t)raw >= a.num_blocks);
    if (!ok && lane == 0) record_error(a.dev_err, TQ_ERR_INDEX, s * a.max_blocks + b);
    return ok ? raw : 0;
  };
  const int o0 = 16 * lane, o1 = o0 + 1024;
  const int kbytes = kf.tile_bytes, vbytes = vf.tile_bytes;
  uint4 nk0 = {0u, 0u, 0u, 0u}, nk1 = nk0, nv0 = nk0, nv1 = nk0;
  bool ok_next = false;
  int b = b0 + wave;
  if (b < b1) {
    const int ph = entry_of(b, ok_next);
    const uint8_t* ksrc = a.k_pages + ((int64_t)ph * a.Hkv + kvh) * kbytes;
    const uint8_t* vsrc = a.v_pages + ((int64_t)ph * a.Hkv + kvh) * vbytes;
    if (o0 < kbytes) nk0 = *reinterpret_cast<const uint4*>(ksrc + o0);
    if (o1 < kbytes) nk1 = *reinterpret_cast<const uint4*>(ksrc + o1);
    if (o0 < vbytes) nv0 = *reinterpret_cast<const uint4*>(vsrc + o0);
    if (o1 < vbytes) nv1 = *reinterpret_cast<const uint4*>(vsrc + o1);
  }
  // (the first block's tiles are requested here, before the query set-up)
  // ---- query: load, K signs, Walsh-Hadamard (fp32), group order
  for (int e = tid; e < 8 * D; e += 64 * kDecWaves) {
    const int g = e / D, c = e - g * D;
    float x = 0.f;
    if (g < G) {
      const int64_t off = ((int64_t)s * a.Hq + kvh * G + g) * D + c;
      x = a.q_f32 ? static_cast<const float*>(a.q)[off]
                  : __uint_as_float((uint32_t)static_cast<const uint16_t*>(a.q)[off] << 16);
      if ((kf.sign_bits[c >> 5] >> (c & 31)) & 1u) x = -x;
    }
    qt[g][c] = x;
  }
  if (tid < 16) {
    cbv[tid] = vf.cb[0][tid];
    vpair[tid] = (uint32_t)vf.cb[0][tid & 3] | ((uint32_t)vf.cb[0][(tid >> 2) & 3] << 16);
  }
  for (int e = tid; e < NG * 256; e += 64 * kDecWaves) {
    const int g = e >> 8, key = e & 255, bits = kf.bits[g];
    const int c0 = key & ((1 << bits) - 1), c1 = (key >> bits) & ((1 << bits) - 1);
    cbpair[g][key] = (uint32_t)kf.cb[g][c0] | ((uint32_t)kf.cb[g][c1] << 16);
  }
  for (int hs = 1; hs < D; hs <<= 1) {
    __syncthreads();
    for (int e = tid; e < 8 * D / 2; e += 64 * kDecWaves) {
      const int g = e / (D / 2), pr = e - g * (D / 2);
      const int i = (pr / hs) * 2 * hs + (pr % hs), j = i + hs;
      const float x0 = qt[g][i], x1 = qt[g][j];
      qt[g][i] = x0 + x1;
      qt[g][j] = x0 - x1;
    }
  }
  __syncthreads();
  for (int e = tid; e < 8 * D; e += 64 * kDecWaves) {
    const int g = e / D, c = e - g * D;
    qg[g][c] = qt[g][kf.ch[c]];
  }
  __syncthreads();
  // ---- projected query u[g][O] = sum_j S[grp][i][j] qg[g][grp M + j], O = grp M + i.
  // The projection rows pass through LDS 32 at a time (coalesced loads, all
  // in flight together; rows padded to M + 1 floats), in the area that holds
  // the wave states after the block loop.
  {
    constexpr int RS = 32;
    float* srows = &st_o[0][0][0];
    static_assert(RS * (M + 1) <= kDecWaves * 8 * D, "projection slice larger than its staging area");
    constexpr int PER = (RS * M / 4 + 64 * kDecWaves - 1) / (64 * kDecWaves);   // float4 per thread per slice
    float4 sv[PER];
    auto fetch_slice = [&](int r0) {
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int e = tid + 64 * kDecWaves * k;
        if (e < RS * M / 4) sv[k] = reinterpret_cast<const float4*>(a.proj + (int64_t)r0 * M)[e];
      }
    };
    fetch_slice(0);
    for (int r0 = 0; r0 < D; r0 += RS) {
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int e = tid + 64 * kDecWaves * k;
        if (e < RS * M / 4) {
          const int r = (4 * e) / M, j = 4 * e - r * M;
          float* dst = srows + r * (M + 1) + j;
          dst[0] = sv[k].x; dst[1] = sv[k].y; dst[2] = sv[k].z; dst[3] = sv[k].w;
        }
      }
      __syncthreads();
      if (r0 + RS < D) fetch_slice(r0 + RS);   // in flight while this slice is used
      {   // 8 heads x 32 rows x 2 halves of the sum = 512 threads; halves added across lanes l, l ^ 1
        static_assert(8 * RS * 2 == 64 * kDecWaves, "one thread per (head, row, half)");
        const int half = tid & 1, rest = tid >> 1;
        const int g = rest / RS, r = rest - g * RS;
        const int O = r0 + r, grp = O / M;
        const float* srow = srows + r * (M + 1) + half * (M / 2);
        const float* qv = qg[g] + grp * M + half * (M / 2);
        float acc = 0.f;
#pragma unroll 16
        for (int j = 0; j < M / 2; ++j) acc = __builtin_fmaf(srow[j], qv[j], acc);
        acc += __shfl_xor(acc, 1);
        if (half == 0) qt[g][O] = acc;
      }
      __syncthreads();
    }
  }
  // ---- per q head: power-of-two scales that put each half of the operand in
  // fp16 range (largest magnitude in [2^14, 2^15)), and the score factors
  {
    const int g = wave;   // 8 waves, 8 heads
    float am = 0.f, au = 0.f;
    for (int c = lane; c < D; c += 64) {
      am = fmaxf(am, fabsf(qg[g][c]));
      au = fmaxf(au, fabsf(qt[g][c]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      am = fmaxf(am, __shfl_xor(am, o));
      au = fmaxf(au, __shfl_xor(au, o));
    }
    int em = 0, eu = 0;
    if (am > 0.f) frexpf(am, &em);
    if (au > 0.f) frexpf(au, &eu);
    const float pm = ldexpf(1.f, 15 - em), pu = ldexpf(1.f, 15 - eu);
    for (int c = lane; c < D; c += 64) {
      qg[g][c] *= pm;
      qt[g][c] *= pu;
    }
    if (lane == 0) {
      wmse[g] = ldexpf(p.f_mse, em - 15);
      wq[g] = ldexpf(p.f_q, eu - 15);
    }
  }
  __syncthreads();
  // ---- B operands: operand t, lane l: column l % 16 (head (l % 16) & 7, high
  // part below 8, low part from 8), channels 32 t + 8 (l / 16) + e
  for (int e = tid; e < 2 * NT * 64; e += 64 * kDecWaves) {
    const int t = e >> 6, l = e & 63;
    const int col = l & 15, g = col & 7;
    const bool lo = col >= 8;
    half8_t v;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = 32 * t + 8 * (l >> 4) + k;
      const float x = c < D ? qg[g][c] : qt[g][c - D];
      const _Float16 hi = (_Float16)x;
      const _Float16 rest16 = (_Float16)(x - (float)hi);
      v[k] = g < G ? (lo ? rest16 : hi) : (_Float16)0.f;
    }
    bop[t][l] = v;
  }
  __syncthreads();

  // ---- blocks of this split, every 8th to each wave
  const int col = lane & 15, gcol = col & 7, ta = lane >> 4;
  const float w_m = wmse[gcol], w_q = wq[gcol];
  // online softmax state per column (exp2 domain): weights 2^(s - m_run +
  // e_run); e_run (the same in every lane) keeps p * n_V * 2^e_run inside
  // fp16's normal range: 15 - ex for the largest V norm so far, 2^(ex-1) <=
  // n < 2^ex (39 before any), so tiny rows keep their precision
  float m_run = -INFINITY, l_run = 0.f;
  int e_run = 39;
  uint32_t v_hi = v_bound_m1(39);
  float4_t o_acc[ND];
#pragma unroll
  for (int u = 0; u < ND; ++u) o_acc[u] = float4_t{0.f, 0.f, 0.f, 0.f};
  uint8_t* kt = ktile[wave];
  uint8_t* vt = vtile[wave];
  const int krb = kf.row_bytes;
  constexpr int m = M;
  for (; b < b1; b += kDecWaves) {
    const bool ok = ok_next;
    wave_fence();   // the previous block's reads of the staging area are done
    if (o0 < kbytes) *reinterpret_cast<uint4*>(kt + o0) = nk0;
    if (o1 < kbytes) *reinterpret_cast<uint4*>(kt + o1) = nk1;
    if (o0 < vbytes) *reinterpret_cast<uint4*>(vt + o0) = nv0;
    if (o1 < vbytes) *reinterpret_cast<uint4*>(vt + o1) = nv1;
    wave_fence();
    if (b + kDecWaves < b1) {
      const int ph = entry_of(b + kDecWaves, ok_next);
      const uint8_t* ksrc = a.k_pages + ((int64_t)ph * a.Hkv + kvh) * kbytes;
      const uint8_t* vsrc = a.v_pages + ((int64_t)ph * a.Hkv + kvh) * vbytes;
      if (o0 < kbytes) nk0 = *reinterpret_cast<const uint4*>(ksrc + o0);
      if (o1 < kbytes) nk1 = *reinterpret_cast<const uint4*>(ksrc + o1);
      if (o0 < vbytes) nv0 = *reinterpret_cast<const uint4*>(vsrc + o0);
      if (o1 < vbytes) nv1 = *reinterpret_cast<const uint4*>(vsrc + o1);
    }
    if (!ok) continue;   // wave-uniform

    // scores: A row r = token sigma(r) = r / 4 + 4 (r % 4), channels 32 t + 8 ta + e;
    // result row 4 ta + i is then token ta + 4 i, the order P.V takes them in
    float4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, accq = acc0;
    const uint8_t* krow = kt + ((col >> 2) + 4 * (col & 3)) * krb;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int P0 = 32 * t + 8 * ta;
      const int g = P0 / m, pos = P0 - g * m;
      const int bits = kf.bits[g];
      const uint8_t* src = krow + kf.grp_byte_off[g] + pos * bits / 8;   // 8 codes = `bits` whole bytes
      uint32_t word = 0;
      if (bits == 4) word = *reinterpret_cast<const uint32_t*>(src);         // 4-byte aligned
      else if (bits == 2) word = *reinterpret_cast<const uint16_t*>(src);    // 2-byte aligned
      else for (int y = 0; y < bits; ++y) word |= (uint32_t)src[y] << (8 * y);
      u32x4_t av;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) av[e2] = cbpair[g][(word >> (2 * bits * e2)) & ((1u << (2 * bits)) - 1u)];
      const half8_t ah = __builtin_bit_cast(half8_t, av);
      if (g == 0) acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bop[t][lane], acc0, 0, 0, 0);
      else acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bop[t][lane], acc1, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int O0 = 32 * t + 8 * ta;
      const int g = O0 / m;
      // residual norm of token sigma(col): norm slot col
      const uint32_t gam = *reinterpret_cast<const uint16_t*>(kt + kf.rnorm_off + 2 * (16 * g + col));
      const uint32_t sb = krow[kf.sign_off + (O0 >> 3)];
      // +-gam in both halves: sign bit 2 e2 of sb to bit 15, bit 2 e2 + 1 to
      // bit 31 (sb | sb << 15 puts them 15 - 2 e2 places below)
      const uint32_t g2 = gam | (gam << 16), spread = sb | (sb << 15);
      u32x4_t av;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) av[e2] = ((spread << (15 - 2 * e2)) & 0x80008000u) | g2;
      accq = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), bop[NT + t][lane], accq, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);   // phase boundary: bounds the registers live across phases
    // lane holds tokens ta + 4 i (norm slots 4 ta + i) of column col; high +
    // low columns summed
    const uint2 nk0 = *reinterpret_cast<const uint2*>(kt + kf.norm_off + 8 * ta);
    const uint2 nk1 = *reinterpret_cast<const uint2*>(kt + kf.norm_off + 32 * (NG - 1) + 8 * ta);
    const uint2 nvv = *reinterpret_cast<const uint2*>(vt + vf.norm_off + 8 * ta);
    // norm products through v_fma_mix (f16 subnormal norms taken as they
    // are, single rounding)
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f0 = acc0[i] + lane_xor<8>(acc0[i], lane);
      const float f1 = acc1[i] + lane_xor<8>(acc1[i], lane);
      const float fq = accq[i] + lane_xor<8>(accq[i], lane);
      const uint32_t k0 = (i >> 1) ? nk0.y : nk0.x;
      float v = (i & 1) ? mul_h<1>(f0, k0) : mul_h<0>(f0, k0);
      if (NG > 1) {
        const uint32_t k1 = (i >> 1) ? nk1.y : nk1.x;
        v = (i & 1) ? fma_h<1>(f1, k1, v) : fma_h<0>(f1, k1, v);
      }
      v = __builtin_fmaf(fq, w_q, v * w_m);
      sc[i] = (16 * b + ta + 4 * i < ctx) ? v : -INFINITY;
    }
    // V norms of the tokens that count; the other rows' bytes may hold
    // anything (set to +0: weight and operand 0)
    uint32_t vx = nvv.x, vy = nvv.y;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (sc[i] == -INFINITY) {
        if (i >> 1) vy &= ~(0xFFFFu << (16 * (i & 1)));
        else vx &= ~(0xFFFFu << (16 * (i & 1)));
      }
    // online softmax per column (exp2 domain)
    float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    bm = fmaxf(bm, lane_xor<16>(bm, lane));
    bm = fmaxf(bm, lane_xor<32>(bm, lane));
    // (no lane leaves here: the matrix-core steps below run with every lane)
    const float m_new = fmaxf(m_run, bm);
    // a V norm too large for e_run lowers it to 15 - ex of the tile's largest
    const u16x2_t mxv = __builtin_elementwise_max(as_u16x2(vx), as_u16x2(vy));
    const bool over = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(mxv, u16x2_t{(uint16_t)v_hi, (uint16_t)v_hi})) != 0u;
    int e_new = e_run;
    if (__builtin_amdgcn_ballot_w64(over)) {
      const uint32_t mh = mxv[0] > mxv[1] ? mxv[0] : mxv[1];
      float vmax = f16_exact<0>(mh);
      vmax = fmaxf(vmax, lane_xor<16>(vmax, lane));
      vmax = fminf(fmaxf(vmax, lane_xor<32>(vmax, lane)), 65504.f);
      const int ex = __builtin_amdgcn_readfirstlane((int)((__float_as_uint(vmax) >> 23) & 0xFF) - 126);
      e_new = 15 - ex < e_run ? 15 - ex : e_run;
      v_hi = v_bound_m1(e_new);
    }
    const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new + (float)(e_new - e_run));
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    m_run = m_new;
    e_run = e_new;
    l_run *= alpha;
#pragma unroll
    for (int u = 0; u < ND; ++u) o_acc[u] *= alpha;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = sc[i] == -INFINITY ? 0.f : exp2f(sc[i] - m_use + (float)e_run);
      l_run += pr[i];
    }
    // p * n_V, each rounded once to fp16
    const half4_t pb = __builtin_bit_cast(half4_t, u32x2_t{mul_h2(pr[0], pr[1], vx), mul_h2(pr[2], pr[3], vy)});
    __builtin_amdgcn_sched_barrier(0);
    // P.V: MFMA u, A row r = dim ND r + u; lane (col, ta) takes run 16 ta + col
    // of the lane-major V plane: VC bytes of each of tokens ta + 4 i, its ND
    // dims' codes, back to back
    const uint8_t* run = vt + (16 * ta + col) * 4 * VC;
    uint32_t vw[4];
    if constexpr (VC == 1) {
      const uint32_t x = *reinterpret_cast<const uint32_t*>(run);
#pragma unroll
      for (int i = 0; i < 4; ++i) vw[i] = (x >> (8 * i)) & 0xFFu;
    } else if constexpr (VC == 2) {
      const uint2 x = *reinterpret_cast<const uint2*>(run);
      vw[0] = x.x & 0xFFFFu; vw[1] = x.x >> 16; vw[2] = x.y & 0xFFFFu; vw[3] = x.y >> 16;
    } else {
      const uint4 x = *reinterpret_cast<const uint4*>(run);
      vw[0] = x.x; vw[1] = x.y; vw[2] = x.z; vw[3] = x.w;
    }
    if constexpr (VB == 2) {
      // two tokens' codes of a dim side by side: each token word's 2-bit
      // codes spread to 4-bit slots, the second token's shifted by 2, so one
      // 4-bit field is the pair-table key of (token i, token i + 1)
      auto spread = [](uint32_t x) -> uint32_t {
        x = (x | (x << 8)) & 0x00FF00FFu;
        x = (x | (x << 4)) & 0x0F0F0F0Fu;
        return (x | (x << 2)) & 0x33333333u;
      };
      const uint32_t w01 = spread(vw[0]) | (spread(vw[1]) << 2);
      const uint32_t w23 = spread(vw[2]) | (spread(vw[3]) << 2);
#pragma unroll
      for (int u = 0; u < ND; ++u) {
        const u32x2_t pv = {vpair[(w01 >> (4 * u)) & 15u], vpair[(w23 >> (4 * u)) & 15u]};
        o_acc[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, pv), pb, o_acc[u], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < ND; ++u) {
        half4_t avv;
#pragma unroll
        for (int i = 0; i < 4; ++i) avv[i] = __builtin_bit_cast(_Float16, cbv[(vw[i] >> (VB * u)) & ((1u << VB) - 1u)]);
        o_acc[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(avv, pb, o_acc[u], 0, 0, 0);
      }
    }
  }
  // ---- wave states: column sums over the 4 token groups
  l_run += lane_xor<16>(l_run, lane);
  l_run += lane_xor<32>(l_run, lane);
  if (col < 8) {
#pragma unroll
    for (int u = 0; u < ND; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) st_o[wave][col][ND * (4 * ta + i) + u] = o_acc[u][i];
    if (ta == 0) {
      st_ml[wave][0][col] = m_run == -INFINITY ? -INFINITY : m_run - (float)e_run;   // the weights' offset
      st_ml[wave][1][col] = l_run;
    }
  }
  __syncthreads();
  // ---- combine, V's 1/sqrt(d), inverse rotation H(.) / sqrt(d) with V signs
  for (int e = tid; e < 8 * D; e += 64 * kDecWaves) {
    const int g = e / D, j = e - g * D;
    float M = -INFINITY;
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, st_ml[w][0][g]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < kDecWaves; ++w) {
        const float mw = st_ml[w][0][g];
        if (mw == -INFINITY) continue;
        const float f = exp2f(mw - M);
        L = __builtin_fmaf(st_ml[w][1][g], f, L);
        O = __builtin_fmaf(st_o[w][g][j], f, O);
      }
    }
    qt[g][j] = L > 0.f ? O / L : 0.f;
  }
  for (int hs = 1; hs < D; hs <<= 1) {
    __syncthreads();
    for (int e = tid; e < 8 * D / 2; e += 64 * kDecWaves) {
      const int g = e / (D / 2), pr = e - g * (D / 2);
      const int i = (pr / hs) * 2 * hs + (pr % hs), j = i + hs;
      const float x0 = qt[g][i], x1 = qt[g][j];
      qt[g][i] = x0 + x1;
      qt[g][j] = x0 - x1;
    }
  }
  __syncthreads();
  const float inv_d = 1.0f / (float)D;
  for (int e = tid; e < G * D; e += 64 * kDecWaves) {
    const int g = e / D, j = e - g * D;
    float M = -INFINITY, L = 0.f;
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, st_ml[w][0][g]);
    if (M != -INFINITY)
      for (int w = 0; w < kDecWaves; ++w)
        if (st_ml[w][0][g] != -INFINITY) L = __builtin_fmaf(st_ml[w][1][g], exp2f(st_ml[w][0][g] - M), L);
    float o = qt[g][j] * inv_d;
    if ((vf.sign_bits[j >> 5] >> (j & 31)) & 1u) o = -o;
    const bool empty = !(L > 0.f);
    if (empty) o = 0.f;
    const int64_t row = (int64_t)s * a.Hq + kvh * G + g;
    const float lse = empty ? -INFINITY : (M + log2f(L)) * 0.6931471805599453f;
    if (P == 1) {
      if (a.out_f32) static_cast<float*>(a.out)[row * D + j] = o;
      else static_cast<uint16_t*>(a.out)[row * D + j] = f32_to_bf16_rne(o);
      if (j == 0 && a.lse) a.lse[row] = lse;
    } else {
      a.part_o[(row * P + sp) * D + j] = o;
      if (j == 0) a.part_lse[row * P + sp] = lse;
    }
  }
}

}  // namespace

tq_status launch_qjl_write(const QjlWriteArgs& a, const DevFormat& kf, hipStream_t st) {
  QjlWriteParams p;
  p.a = a;
  p.f = kf;
  const int64_t rows = a.num_tokens * a.H;
  if (rows == 0) return TQ_OK;
  const int64_t wgs = std::min<int64_t>((rows + kWriteWaves - 1) / kWriteWaves, (int64_t)device_cus() * 4);
  const dim3 grid((unsigned)wgs);
  if (kf.d == 128) {
    if (a.f32) hipLaunchKernelGGL((qjl_write_kernel<128, true>), grid, dim3(64 * kWriteWaves), 0, st, p);
    else hipLaunchKernelGGL((qjl_write_kernel<128, false>), grid, dim3(64 * kWriteWaves), 0, st, p);
  } else {
    if (a.f32) hipLaunchKernelGGL((qjl_write_kernel<64, true>), grid, dim3(64 * kWriteWaves), 0, st, p);
    else hipLaunchKernelGGL((qjl_write_kernel<64, false>), grid, dim3(64 * kWriteWaves), 0, st, p);
  }
  return launch_status("tq_write_kv QJL launch");
}

tq_status launch_qjl_decode(const QjlDecodeArgs& a, const DevFormat& kf, const DevFormat& vf, hipStream_t st) {
  if (kf.tile_bytes > kKTileMax || vf.tile_bytes > kVTileMax)
    return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "QJL decode: tile larger than the staging area");
  if (a.G < 1 || a.G > 8) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "QJL decode: more than 8 q heads per kv head");
  QjlDecParams p;
  p.a = a;
  p.kf = kf;
  p.vf = vf;
  const double log2e = 1.4426950408889634;
  const double d = kf.d, m = kf.m;
  p.f_mse = (float)((double)a.scale * log2e / sqrt(m * d));
  p.f_q = (float)((double)a.scale * log2e * sqrt(M_PI / 2.0) / (m * sqrt(d)));
  const int64_t n_wg = (int64_t)a.S * a.Hkv * a.P;
  if (n_wg == 0) return TQ_OK;
  if (n_wg >= ((int64_t)1 << 31)) return set_error(TQ_ERR_VALUE, "QJL decode: too many workgroups");
  const dim3 grid((unsigned)n_wg);
  const dim3 block(64 * kDecWaves);
  if (vf.ng != 1 || (vf.bits[0] != 2 && vf.bits[0] != 4) || vf.chunk * 16 != vf.row_bytes)
    return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "QJL decode: V must be one group of 2 or 4 bits");
#define TQ_QJL(DD, NGG, VBB)                                                     \
  if (kf.d == DD && kf.ng == NGG && vf.bits[0] == VBB) {                        \
    hipLaunchKernelGGL((qjl_decode_kernel<DD, NGG, VBB>), grid, block, 0, st, p); \
    return launch_status("tq_decode_paged QJL launch");                          \
  }
  TQ_QJL(128, 1, 4) TQ_QJL(128, 1, 2) TQ_QJL(128, 2, 4) TQ_QJL(128, 2, 2)
  TQ_QJL(64, 1, 4) TQ_QJL(64, 1, 2) TQ_QJL(64, 2, 4) TQ_QJL(64, 2, 2)
#undef TQ_QJL
  return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "QJL decode: no kernel for this format");
}

}  // namespace tq
