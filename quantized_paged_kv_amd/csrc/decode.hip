// Paged decode attention over packed, rotated, codebook-quantised K/V pages,
// plus the log-sum-exp merge of split partials.
//
// [D "Serving Route Design"]: block tables map logical to physical blocks;
// K rows are read inside the score computation and V rows are dequantised
// inside the accumulation; the workspace is bounded by the runtime shape.
// [D "System Invariants"]: production routes consume packed history (no dense
// K/V tensor is ever formed); unsupported formats raise.
//
// Work decomposition.  One workgroup (8 waves) owns one item = (sequence,
// kv head, chunk of C logical blocks); the 8 waves take the chunk's blocks
// round-robin, each keeping its own online-softmax state, and merge through
// LDS at the end.  Items are numbered sequence-major over the chunks that a
// sequence actually has, so no workgroup is spent on empty chunks, and the
// workgroup-to-item map places the kv heads of one chunk on one XCD (the
// heads of a physical block are adjacent in the pool and share cache lines).
//
// Inner loop (per wave, per 16-token block), all in the rotated domain:
//   q.K:  v_mfma_f32_16x16x32_f16, A = dequantised K rows (16 tokens x 32
//         channels, codebook values exact in fp16), B = rotated q split into
//         an fp16 high and low part (columns 0-7 high, 8-15 low, one column
//         per q head of the GQA group), so the score keeps ~fp32 accuracy.
//         Token order inside the tile is sigma(4a + e) = a + 4e, which makes
//         the score accumulator layout the B operand of P.V unchanged.
//   softmax: exp2 domain, running max per q head shared by the four lanes
//         that hold that head's 16 scores; rescale only when the max grows.
//   P.V:  v_mfma_f32_16x16x16_f16, A = dequantised V (dims x tokens), B =
//         p * (V norm) in fp16, accumulators fp32.
// Codebook lookups use byte-indexed LDS tables replicated across banks
// (one v_perm builds the address from a packed byte and the lane's copy).
// Epilogue: inverse rotation of the output once per head (Walsh-Hadamard
// across the wave, signs, 1/sqrt(d)), LDS merge of the 8 wave states, then
// either the final output or a split partial.
#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kLutBytes = 65536;    // 256 entries x 256 B (two halves)
constexpr int kLut3Bytes = 8192;    // 64 entries x 32 copies x 4 B
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum KKind { K4 = 0, K2 = 1, KM43 = 2 };
enum VKind { V4 = 0, V2 = 1 };

struct DecodeParams {
  const void* q;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* lse;
  float* part_o;     // [S][Hq][P][D]
  float* part_lse;   // [S][Hq][P]
  int32_t* dev_err;
  int64_t num_blocks;
  int32_t S, Hq, Hkv, G, max_blocks, P, C;
  int32_t k_tile, v_tile, k_norm_off, v_norm_off;
  int32_t n_items_bound;
  float score_mul;   // scale * log2(e) / (sqrt(D) * sqrt(m_K))
  float v_mul;       // 1 / sqrt(m_V)
  uint32_t v_signs[4];
  uint32_t k_signs[4];
  uint16_t half_cb[2][16];   // codebook of the table in each LUT half
  int32_t half_kind[2];      // 0 none, 4 = nibble table, 2 = crumb table
  uint16_t k3_cb[8];         // 3-bit codebook of the mixed K low group
  uint8_t k_ch[128];
  int32_t v_half;            // LUT half that V reads
  int32_t q_f32, out_f32;
};

__device__ __forceinline__ void record_error(int32_t* err, int32_t code, int32_t pos) {
  if (err && atomicCAS(err, 0, code) == 0) atomicExch(err + 1, pos);
}

__device__ __forceinline__ uint32_t lut_addr(uint32_t packed, uint32_t lane_off, int byte) {
  // [lane_off.byte0, packed.byte(byte), 0, 0] = byte * 256 + lane_off
  return __builtin_amdgcn_perm(packed, lane_off, 0x0C0C0400u | ((uint32_t)byte << 8));
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* lds, uint32_t addr) {
  return *reinterpret_cast<const uint32_t*>(lds + addr);
}
__device__ __forceinline__ uint2 lds_u64(const uint8_t* lds, uint32_t addr) {
  return *reinterpret_cast<const uint2*>(lds + addr);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float row_ror8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t half2_bits(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

template <int D, int KK, int VK>
struct Cfg {
  static constexpr int R = D / 16;                       // dims per lane-row in P.V
  static constexpr int NQK = D / 32;                     // q.K MFMAs per block
  static constexpr int KROW = KK == K4 ? D / 2 : (KK == K2 ? D / 4 : (D / 2) * 4 / 8 + (D / 2) * 3 / 8);
  static constexpr int VROW = VK == V4 ? D / 2 : D / 4;
  static constexpr int VLANE = VK == V4 ? D / 32 : D / 64;  // bytes per lane per token in V
  static constexpr bool MIXED = KK == KM43;
  static constexpr int LDS_BYTES = kLutBytes + (MIXED ? kLut3Bytes : 0);
};

// Per-block raw loads of one wave.
template <int D, int KK, int VK>
struct Tile {
  uint32_t k[4];      // packed K bits of this lane (up to 16 B)
  uint32_t k_lo[2];   // mixed: low-group bits (aligned 8 B window)
  uint2 kn[2];        // K norms of the lane's 4 tokens, per group
  uint32_t v[4];      // packed V bits of the lane's 4 tokens
  uint2 vn;           // V norms
};

template <int D, int KK, int VK>
__device__ __forceinline__ void load_tile(Tile<D, KK, VK>& t, const uint8_t* kt, const uint8_t* vt, int tokK, int c,
                                          int a, int i, int k_norm_off, int v_norm_off) {
  using C = Cfg<D, KK, VK>;
  if constexpr (KK == K4) {
    if constexpr (D == 128) {
      const uint4 x = *reinterpret_cast<const uint4*>(kt + tokK * C::KROW + 16 * c);
      t.k[0] = x.x; t.k[1] = x.y; t.k[2] = x.z; t.k[3] = x.w;
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(kt + tokK * C::KROW + 8 * c);
      t.k[0] = x.x; t.k[1] = x.y;
    }
  } else if constexpr (KK == K2) {
    if constexpr (D == 128) {
      const uint2 x = *reinterpret_cast<const uint2*>(kt + tokK * C::KROW + 8 * c);
      t.k[0] = x.x; t.k[1] = x.y;
    } else {
      t.k[0] = *reinterpret_cast<const uint32_t*>(kt + tokK * C::KROW + 4 * c);
    }
  } else {
    constexpr int HB = D / 4;             // high group bytes per row (4-bit, D/2 channels)
    constexpr int LB = 3 * D / 64;        // low group bytes per lane (3-bit, D/8 channels)
    if constexpr (D == 128) {
      const uint2 x = *reinterpret_cast<const uint2*>(kt + tokK * C::KROW + 8 * c);
      t.k[0] = x.x; t.k[1] = x.y;
    } else {
      t.k[0] = *reinterpret_cast<const uint32_t*>(kt + tokK * C::KROW + 4 * c);
    }
    const int lo_off = tokK * C::KROW + HB + LB * c;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(kt + (lo_off & ~3));
    t.k_lo[0] = w[0];
    t.k_lo[1] = w[1];
  }
  t.kn[0] = *reinterpret_cast<const uint2*>(kt + k_norm_off + 8 * a);
  if constexpr (C::MIXED) t.kn[1] = *reinterpret_cast<const uint2*>(kt + k_norm_off + 32 + 8 * a);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint8_t* row = vt + (a + 4 * r) * C::VROW;
    if constexpr (C::VLANE == 4) t.v[r] = *reinterpret_cast<const uint32_t*>(row + 4 * i);
    else if constexpr (C::VLANE == 2) t.v[r] = *reinterpret_cast<const uint16_t*>(row + 2 * i);
    else t.v[r] = row[i];
  }
  t.vn = *reinterpret_cast<const uint2*>(vt + v_norm_off + 8 * a);
}

template <int D, int KK, int VK>
__global__ __launch_bounds__(kThreads, 4) void decode_kernel(DecodeParams p) {
  using C = Cfg<D, KK, VK>;
  constexpr int R = C::R;
  constexpr int NQK = C::NQK;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];
  __shared__ float qbuf[8][D];
  __shared__ int qexp[8];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  // ---- which item: XCD-aware order, then sequence-major scan of chunk counts
  const int nwg = gridDim.x;
  const int per_xcd = (nwg + 7) >> 3;
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  int s = -1, part = 0, kvh = 0, ctx = 0;
  {
    int before = 0;
    for (int base = 0; base < p.S && s < 0; base += 64) {
      const int sq = base + lane;
      int cnt = 0, c_l = 0;
      if (sq < p.S) {
        c_l = p.context_lens[sq];
        const int cap = p.max_blocks * 16;
        if (c_l < 0 || c_l > cap) {
          if (blockIdx.x == 0 && wave == 0) record_error(p.dev_err, TQ_ERR_INDEX, -1 - sq);
          c_l = c_l < 0 ? 0 : cap;
        }
        const int nb = (c_l + 15) >> 4;
        int np = (nb + p.C - 1) / p.C;
        if (np < 1) np = 1;
        cnt = np * p.Hkv;
      }
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      const int excl = incl - cnt;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(sq < p.S && item >= before + excl && item < before + incl);
      if (hit) {
        const int src = __builtin_ctzll(hit);
        const int e0 = __shfl(excl, src);
        s = base + src;
        ctx = __shfl(c_l, src);
        const int r = item - before - e0;
        part = r / p.Hkv;
        kvh = r % p.Hkv;
      }
      before += __shfl(incl, 63);
    }
  }
  if (s < 0) return;  // uniform across the workgroup

  const int nb_seq = (ctx + 15) >> 4;
  const int b_begin = part * p.C;
  int b_end = b_begin + p.C;
  if (b_end > nb_seq) b_end = nb_seq;

  // ---- LDS tables: byte-indexed, two halves of 128 B per entry
  for (int idx = tid; idx < kLutBytes / 4; idx += kThreads) {
    const int e = idx >> 6, w = idx & 63, h = w >> 5;
    const int kind = p.half_kind[h];
    uint32_t val = 0;
    if (kind == 4) {
      val = (uint32_t)p.half_cb[h][e & 15] | ((uint32_t)p.half_cb[h][e >> 4] << 16);
    } else if (kind == 2) {
      val = (w & 1) ? ((uint32_t)p.half_cb[h][(e >> 4) & 3] | ((uint32_t)p.half_cb[h][e >> 6] << 16))
                    : ((uint32_t)p.half_cb[h][e & 3] | ((uint32_t)p.half_cb[h][(e >> 2) & 3] << 16));
    }
    reinterpret_cast<uint32_t*>(lds)[idx] = val;
  }
  if constexpr (C::MIXED) {
    for (int idx = tid; idx < kLut3Bytes / 4; idx += kThreads) {
      const int e = idx >> 5;
      reinterpret_cast<uint32_t*>(lds + kLutBytes)[idx] = (uint32_t)p.k3_cb[e & 7] | ((uint32_t)p.k3_cb[e >> 3] << 16);
    }
  }

  // ---- rotate the G q heads once: qbuf[g][ch] = (H (s_K * q))[ch], fp32
  if (wave == 0) {
    constexpr int PER = D / 8;              // channels per lane, 8 lanes per head
    const int g = lane >> 3, l8 = lane & 7;
    float x[PER];
    const int hq = kvh * p.G + g;
    const bool live = g < p.G;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int chn = l8 * PER + e;
      float v = 0.f;
      if (live) {
        const int64_t off = ((int64_t)s * p.Hq + hq) * D + chn;
        v = p.q_f32 ? static_cast<const float*>(p.q)[off] : bf16_to_f32(static_cast<const uint16_t*>(p.q)[off]);
        if ((p.k_signs[chn >> 5] >> (chn & 31)) & 1u) v = -v;
      }
      x[e] = v;
    }
#pragma unroll
    for (int h = 1; h < PER; h <<= 1) {
#pragma unroll
      for (int e = 0; e < PER; ++e)
        if ((e & h) == 0) {
          const float a0 = x[e], b0 = x[e + h];
          x[e] = a0 + b0;
          x[e + h] = a0 - b0;
        }
    }
#pragma unroll
    for (int k = 1; k < 8; k <<= 1) {
      const bool up = (l8 & k) != 0;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float o = __shfl_xor(x[e], k);
        x[e] = up ? (o - x[e]) : (x[e] + o);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      qbuf[g][l8 * PER + e] = x[e];
      amax = fmaxf(amax, fabsf(x[e]));
    }
#pragma unroll
    for (int k = 1; k < 8; k <<= 1) amax = fmaxf(amax, __shfl_xor(amax, k));
    if (l8 == 0) {
      int ex = 0;
      if (amax > 0.f) {
        frexpf(amax, &ex);
      }
      qexp[g] = 15 - ex;   // amax * 2^(15-ex) in [2^14, 2^15)
    }
  }
  __syncthreads();

  // ---- per-lane roles
  const int j = lane & 15;          // MFMA column: q head j & 7, high (j < 8) or low part
  const int a = lane >> 4;          // token group: tokens a, a+4, a+8, a+12 of a block
  const int gq = j & 7;
  const bool lo_part = j >= 8;
  const bool col_live = gq < p.G;
  const int kq = qexp[gq];
  const float q_pow = ldexpf(1.0f, kq);
  const float w_col = ldexpf(p.score_mul, -kq);

  // B operands of q.K: MFMA t covers listed channels of this lane's range
  half8_t qb[NQK];
#pragma unroll
  for (int t = 0; t < NQK; ++t) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int pos;
      if constexpr (C::MIXED) {
        constexpr int m = D / 2;
        constexpr int per_g = NQK / 2;
        const int grp = t / per_g, u = t % per_g;
        pos = grp * m + a * (m / 4) + 8 * u + e;
      } else {
        pos = a * (D / 4) + 8 * t + e;
      }
      const int chn = C::MIXED ? (int)p.k_ch[pos] : pos;
      const float v = col_live ? qbuf[gq][chn] * q_pow : 0.f;
      const _Float16 hi = (_Float16)v;
      const _Float16 lo = (_Float16)(v - (float)hi);
      qb[t][e] = lo_part ? lo : hi;
    }
  }
  __syncthreads();  // qbuf is not read again; tables are complete

  // ---- lane-dependent table offsets
  const uint32_t off4_k = (uint32_t)(lane & 31) * 4u;                      // K nibble table, half 0
  const uint32_t off2_k = (uint32_t)(lane & 15) * 8u;                      // K crumb table, half 0
  const uint32_t off_v4 = (uint32_t)p.v_half * 128u + (uint32_t)(lane & 31) * 4u;
  const uint32_t off_v2 = (uint32_t)p.v_half * 128u + (uint32_t)(lane & 15) * 8u;
  const uint32_t off3 = (uint32_t)kLutBytes + (uint32_t)(lane & 31) * 4u;

  // token of this lane's K row: sigma(j) = j/4 + 4*(j%4)
  const int tokK = (j >> 2) + 4 * (j & 3);

  const uint8_t* k_head = p.k_pages + (int64_t)kvh * p.k_tile;
  const uint8_t* v_head = p.v_pages + (int64_t)kvh * p.v_tile;
  const int64_t k_blk_stride = (int64_t)p.Hkv * p.k_tile;
  const int64_t v_blk_stride = (int64_t)p.Hkv * p.v_tile;
  const int32_t* bt_row = p.block_tables + (int64_t)s * p.max_blocks;

  float m_run = -INFINITY, l_run = 0.f;
  float4_t o_acc[R];
#pragma unroll
  for (int u = 0; u < R; ++u) o_acc[u] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int nbw = (b_end - b_begin - wave + kWaves - 1) / kWaves;  // blocks of this wave
  for (int chunk0 = 0; chunk0 < nbw; chunk0 += 64) {
    const int cnt = (nbw - chunk0) < 64 ? (nbw - chunk0) : 64;
    int bt_reg = 0;
    if (lane < cnt) bt_reg = bt_row[b_begin + wave + kWaves * (chunk0 + lane)];

    Tile<D, KK, VK> cur, nxt;
    auto tile_ptrs = [&](int it, const uint8_t*& kt, const uint8_t*& vt) -> bool {
      const int phys = __builtin_amdgcn_readlane(bt_reg, it);
      const bool ok = phys >= 0 && (int64_t)phys < p.num_blocks;
      const int64_t ph = ok ? phys : 0;
      kt = k_head + ph * k_blk_stride;
      vt = v_head + ph * v_blk_stride;
      return ok;
    };
    const uint8_t *kt0, *vt0;
    bool ok_cur = tile_ptrs(0, kt0, vt0);
    load_tile<D, KK, VK>(cur, kt0, vt0, tokK, a, a, j, p.k_norm_off, p.v_norm_off);

    for (int it = 0; it < cnt; ++it) {
      bool ok_nxt = false;
      if (it + 1 < cnt) {
        const uint8_t *kt1, *vt1;
        ok_nxt = tile_ptrs(it + 1, kt1, vt1);
        load_tile<D, KK, VK>(nxt, kt1, vt1, tokK, a, a, j, p.k_norm_off, p.v_norm_off);
      }
      const int b = b_begin + wave + kWaves * (chunk0 + it);
      if (!ok_cur && lane == 0) record_error(p.dev_err, TQ_ERR_INDEX, s * p.max_blocks + b);

      // -------- q.K on the matrix cores
      float4_t acc0 = {0.f, 0.f, 0.f, 0.f};
      float4_t acc1 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (KK == K4) {
#pragma unroll
        for (int t = 0; t < NQK; ++t) {
          u32x4_t av;
#pragma unroll
          for (int by = 0; by < 4; ++by) av[by] = lds_u32(lds, lut_addr(cur.k[t], off4_k, by));
          const half8_t A = __builtin_bit_cast(half8_t, av);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qb[t], acc0, 0, 0, 0);
        }
      } else if constexpr (KK == K2) {
#pragma unroll
        for (int t = 0; t < NQK; ++t) {
          const uint2 x0 = lds_u64(lds, lut_addr(cur.k[t >> 1], off2_k, 2 * (t & 1)));
          const uint2 x1 = lds_u64(lds, lut_addr(cur.k[t >> 1], off2_k, 2 * (t & 1) + 1));
          const u32x4_t av = {x0.x, x0.y, x1.x, x1.y};
          const half8_t A = __builtin_bit_cast(half8_t, av);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qb[t], acc0, 0, 0, 0);
        }
      } else {
        constexpr int per_g = NQK / 2;
        // high group: 4-bit nibbles
#pragma unroll
        for (int u = 0; u < per_g; ++u) {
          u32x4_t av;
#pragma unroll
          for (int by = 0; by < 4; ++by) av[by] = lds_u32(lds, lut_addr(cur.k[u], off4_k, by));
          const half8_t A = __builtin_bit_cast(half8_t, av);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qb[u], acc0, 0, 0, 0);
        }
        // low group: 3-bit indices, looked up in pairs (6-bit keys)
        {
          constexpr int LB = 3 * D / 64;
          const int lo_off = tokK * C::KROW + D / 4 + LB * a;
          const uint64_t win = ((uint64_t)cur.k_lo[1] << 32 | cur.k_lo[0]) >> ((lo_off & 3) * 8);
#pragma unroll
          for (int u = 0; u < per_g; ++u) {
            u32x4_t av;
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
              const uint32_t key = (uint32_t)(win >> (6 * (4 * u + pr))) & 63u;
              av[pr] = lds_u32(lds, (key << 7) | off3);
            }
            const half8_t A = __builtin_bit_cast(half8_t, av);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qb[per_g + u], acc1, 0, 0, 0);
          }
        }
      }

      // -------- scores of this lane's 4 tokens for q head gq (exp2 domain)
      const int tok0 = 16 * b;
      float sc[4];
      {
        const uint32_t kn0[2] = {cur.kn[0].x, cur.kn[0].y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float full0 = acc0[e] + row_ror8(acc0[e]);
          const _Float16 n0 = __builtin_bit_cast(_Float16, (uint16_t)(kn0[e >> 1] >> (16 * (e & 1))));
          float v = full0 * ((float)n0 * w_col);
          if constexpr (C::MIXED) {
            const uint32_t kn1[2] = {cur.kn[1].x, cur.kn[1].y};
            const float full1 = acc1[e] + row_ror8(acc1[e]);
            const _Float16 n1 = __builtin_bit_cast(_Float16, (uint16_t)(kn1[e >> 1] >> (16 * (e & 1))));
            v += full1 * ((float)n1 * w_col);
          }
          const bool valid = ok_cur && col_live && (tok0 + a + 4 * e) < ctx;
          sc[e] = valid ? v : -INFINITY;
        }
      }
      float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float m_new = fmaxf(m_run, bm);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {
        const float alpha = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // m_run = -inf -> 0
        l_run *= alpha;
#pragma unroll
        for (int u = 0; u < R; ++u) o_acc[u] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pr[e] = __builtin_amdgcn_exp2f(sc[e] - m_use);
        l_run += pr[e];
      }
      half4_t pb;
      {
        const uint32_t vn[2] = {cur.vn.x, cur.vn.y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const _Float16 nv = __builtin_bit_cast(_Float16, (uint16_t)(vn[e >> 1] >> (16 * (e & 1))));
          const float pv = (sc[e] == -INFINITY) ? 0.f : pr[e] * ((float)nv * p.v_mul);
          pb[e] = (_Float16)pv;
        }
      }

      // -------- P.V on the matrix cores: A = V (dims x tokens) per MFMA u
      if constexpr (VK == V4) {
        constexpr int NB = D / 32;  // bytes per token in this lane (2 dims each)
#pragma unroll
        for (int k = 0; k < NB; ++k) {
          uint32_t lk[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) lk[r] = lds_u32(lds, lut_addr(cur.v[r], off_v4, k));
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const uint32_t sel = hh ? 0x07060302u : 0x05040100u;
            const u32x2_t av = {__builtin_amdgcn_perm(lk[1], lk[0], sel), __builtin_amdgcn_perm(lk[3], lk[2], sel)};
            const half4_t A = __builtin_bit_cast(half4_t, av);
            o_acc[2 * k + hh] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, pb, o_acc[2 * k + hh], 0, 0, 0);
          }
        }
      } else {
        constexpr int NBY = D / 64;  // bytes per token in this lane (4 dims each)
#pragma unroll
        for (int k = 0; k < NBY; ++k) {
          uint2 lk[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) lk[r] = lds_u64(lds, lut_addr(cur.v[r], off_v2, k));
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t w0 = (t >> 1) ? lk[0].y : lk[0].x;
            const uint32_t w1 = (t >> 1) ? lk[1].y : lk[1].x;
            const uint32_t w2 = (t >> 1) ? lk[2].y : lk[2].x;
            const uint32_t w3 = (t >> 1) ? lk[3].y : lk[3].x;
            const u32x2_t av = {__builtin_amdgcn_perm(w1, w0, sel), __builtin_amdgcn_perm(w3, w2, sel)};
            const half4_t A = __builtin_bit_cast(half4_t, av);
            o_acc[4 * k + t] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, pb, o_acc[4 * k + t], 0, 0, 0);
          }
        }
      }
      cur = nxt;
      ok_cur = ok_nxt;
    }
  }

  // ---- wave epilogue: full row sum, inverse rotation of this lane's dims
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  float y[4 * R];
#pragma unroll
  for (int u = 0; u < R; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) y[R * e + u] = o_acc[u][e];
#pragma unroll
  for (int h = 1; h < 4 * R; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 4 * R; ++e)
      if ((e & h) == 0) {
        const float a0 = y[e], b0 = y[e + h];
        y[e] = a0 + b0;
        y[e + h] = a0 - b0;
      }
  }
#pragma unroll
  for (int k = 16; k < 64; k <<= 1) {
    const bool up = (lane & k) != 0;
#pragma unroll
    for (int e = 0; e < 4 * R; ++e) {
      const float o = __shfl_xor(y[e], k);
      y[e] = up ? (o - y[e]) : (y[e] + o);
    }
  }

  __syncthreads();  // every wave is done with the tables: reuse LDS for the merge
  float* mo = reinterpret_cast<float*>(lds);               // [kWaves][8][D]
  float* mm = mo + kWaves * 8 * D;                          // [kWaves][8]
  float* ml = mm + kWaves * 8;                              // [kWaves][8]
  if (!lo_part) {
#pragma unroll
    for (int e = 0; e < 4 * R; ++e) {
      const int dim = 4 * R * a + e;
      const float sg = ((p.v_signs[dim >> 5] >> (dim & 31)) & 1u) ? -1.f : 1.f;
      mo[(wave * 8 + gq) * D + dim] = y[e] * sg;
    }
    if (a == 0) {
      mm[wave * 8 + gq] = m_run;
      ml[wave * 8 + gq] = l_run;
    }
  }
  __syncthreads();

  // ---- merge the 8 wave states and write the result
  const float inv_sqrt_d = D == 128 ? 0.08838834764831845f : 0.125f;
  for (int idx = tid; idx < p.G * D; idx += kThreads) {
    const int g = idx / D, dim = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mm[w * 8 + g]);
    float den = 0.f, num = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = mm[w * 8 + g];
        const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        den += f * ml[w * 8 + g];
        num += f * mo[(w * 8 + g) * D + dim];
      }
    }
    const bool empty = !(den > 0.f);
    const float o = empty ? 0.f : num / den * inv_sqrt_d;
    const float lse = empty ? -INFINITY : (M + log2f(den)) * kLn2;
    const int hq = kvh * p.G + g;
    if (p.P == 1) {
      const int64_t off = ((int64_t)s * p.Hq + hq) * D + dim;
      if (p.out_f32) static_cast<float*>(p.out)[off] = o;
      else static_cast<uint16_t*>(p.out)[off] = f32_to_bf16_rne(o);
      if (dim == 0 && p.lse) p.lse[(int64_t)s * p.Hq + hq] = lse;
    } else {
      const int64_t row = ((int64_t)s * p.Hq + hq) * p.P + part;
      p.part_o[row * D + dim] = o;
      if (dim == 0) p.part_lse[row] = lse;
    }
  }
}

// ----------------------------------------------------------------- merge
// One wave per (sequence, head).  n_valid(s) partials are read (all P for
// the generic entry point; the chunks the sequence has for the decode).
struct MergeParams {
  const float* part_o;
  const float* part_lse;
  void* out;
  float* lse;
  const int32_t* context_lens;  // NULL: all P partials
  int32_t S, H, P, D, C, max_blocks, out_f32;
};

__global__ __launch_bounds__(64) void merge_kernel(MergeParams p) {
  const int sh = blockIdx.x;
  const int s = sh / p.H;
  const int lane = threadIdx.x;
  int n = p.P;
  if (p.context_lens) {
    int c = p.context_lens[s];
    const int cap = p.max_blocks * 16;
    c = c < 0 ? 0 : (c > cap ? cap : c);
    const int nb = (c + 15) >> 4;
    n = (nb + p.C - 1) / p.C;
    if (n < 1) n = 1;
    if (n > p.P) n = p.P;
  }
  const float* lse_p = p.part_lse + (int64_t)sh * p.P;
  const float* o_p = p.part_o + (int64_t)sh * p.P * p.D;
  float M = -INFINITY;
  for (int i = lane; i < n; i += 64) M = fmaxf(M, lse_p[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float acc[2] = {0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {
    for (int i = 0; i < n; ++i) {
      const float li = lse_p[i];
      const float w = (li == -INFINITY) ? 0.f : expf(li - M);
      den += w;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int dim = lane + 64 * r;
        if (dim < p.D) acc[r] += w * o_p[(int64_t)i * p.D + dim];
      }
    }
  }
  const bool empty = !(den > 0.f);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int dim = lane + 64 * r;
    if (dim >= p.D) continue;
    const float o = empty ? 0.f : acc[r] / den;
    const int64_t off = (int64_t)sh * p.D + dim;
    if (p.out_f32) static_cast<float*>(p.out)[off] = o;
    else static_cast<uint16_t*>(p.out)[off] = f32_to_bf16_rne(o);
  }
  if (lane == 0 && p.lse) p.lse[sh] = empty ? -INFINITY : M + logf(den);
}

template <int D, int KK, int VK>
void launch_decode(const DecodeParams& p, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<D, KK, VK>), dim3(grid), dim3(kThreads), 0, st, p);
}

int format_kind_k(const tq_format* f) {
  if (f->num_groups == 1 && f->group_bits[0] == 4) return K4;
  if (f->num_groups == 1 && f->group_bits[0] == 2) return K2;
  if (f->num_groups == 2 && f->group_bits[0] == 4 && f->group_bits[1] == 3) return KM43;
  return -1;
}

int format_kind_v(const tq_format* f) {
  if (f->num_groups == 1 && f->group_bits[0] == 4) return V4;
  if (f->num_groups == 1 && f->group_bits[0] == 2) return V2;
  return -1;
}

}  // namespace
}  // namespace tq

using namespace tq;

extern "C" tq_status tq_split_merge(const float* part_out, const float* part_lse, int32_t num_seqs,
                                    int32_t num_heads, int32_t num_splits, int32_t head_dim, void* out,
                                    tq_dtype out_dtype, float* lse, tq_stream_t stream) {
  if (num_seqs < 0 || num_heads <= 0 || num_splits <= 0) return set_error(TQ_ERR_VALUE, "bad merge shape");
  if (head_dim != 64 && head_dim != 128) return set_error(TQ_ERR_VALUE, "head_dim must be 64 or 128");
  if (out_dtype != TQ_BF16 && out_dtype != TQ_F32) return set_error(TQ_ERR_VALUE, "out_dtype must be BF16 or F32");
  if (num_seqs == 0) return TQ_OK;
  if (!part_out || !part_lse || !out) return set_error(TQ_ERR_VALUE, "NULL merge buffer");
  MergeParams mp = {part_out, part_lse, out, lse, nullptr, num_seqs, num_heads, num_splits, head_dim, 1, 1,
                    out_dtype == TQ_F32};
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(num_seqs * num_heads)), dim3(64), 0,
                     reinterpret_cast<hipStream_t>(stream), mp);
  return launch_status("tq_split_merge launch");
}

extern "C" tq_status tq_decode_paged(const void* q, tq_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t num_kv_heads, const uint8_t* k_pages, const uint8_t* v_pages,
                                     int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                                     const tq_format* kfmt, const tq_format* vfmt, float scale,
                                     int32_t num_splits, void* workspace, uint64_t workspace_bytes, void* out,
                                     tq_dtype out_dtype, float* lse, int32_t* dev_err, tq_stream_t stream) {
  tq_status st = check_format(kfmt, "K");
  if (st != TQ_OK) return st;
  st = check_format(vfmt, "V");
  if (st != TQ_OK) return st;
  if (kfmt->head_dim != vfmt->head_dim) return set_error(TQ_ERR_VALUE, "K and V head_dim differ");
  if (q_dtype != TQ_BF16 && q_dtype != TQ_F32) return set_error(TQ_ERR_VALUE, "q_dtype must be BF16 or F32");
  if (out_dtype != TQ_BF16 && out_dtype != TQ_F32) return set_error(TQ_ERR_VALUE, "out_dtype must be BF16 or F32");
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return set_error(TQ_ERR_VALUE, "shape arguments must be positive");
  if (num_q_heads % num_kv_heads != 0) return set_error(TQ_ERR_VALUE, "num_q_heads must be a multiple of num_kv_heads");
  if (num_splits <= 0) return set_error(TQ_ERR_VALUE, "num_splits must be >= 1");
  if (block_size != TQ_BLOCK_SIZE) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "block_size must be 16");
  const int G = num_q_heads / num_kv_heads;
  if (G > 8) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "more than 8 q heads per kv head");
  const int kk = format_kind_k(kfmt), vk = format_kind_v(vfmt);
  if (kk < 0) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "no decode kernel for this K format (served: 4-bit, 2-bit, 4+3-bit groups)");
  if (vk < 0) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "no decode kernel for this V format (served: 4-bit, 2-bit)");
  const int D = kfmt->head_dim;
  if (kk == KM43 && D != 128 && D != 64) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "mixed K needs head_dim 64 or 128");
  if (num_seqs == 0) return TQ_OK;
  if (!q || !k_pages || !v_pages || !block_tables || !context_lens || !out)
    return set_error(TQ_ERR_VALUE, "NULL required pointer");
  uint64_t need = 0;
  tq_decode_workspace_bytes(num_seqs, num_q_heads, D, num_splits, &need);
  if (workspace_bytes < need || (need && !workspace))
    return set_error(TQ_ERR_VALUE, "workspace too small: need " + std::to_string(need) + " bytes");
  const int64_t items = (int64_t)num_seqs * num_splits * num_kv_heads;
  if (items >= (1ll << 31) / 2) return set_error(TQ_ERR_VALUE, "too many decode items");

  DecodeParams p = {};
  p.q = q;
  p.k_pages = k_pages;
  p.v_pages = v_pages;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.lse = lse;
  p.dev_err = dev_err;
  p.num_blocks = num_blocks;
  p.S = num_seqs;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.G = G;
  p.max_blocks = max_blocks_per_seq;
  p.P = num_splits;
  p.C = (max_blocks_per_seq + num_splits - 1) / num_splits;
  p.k_tile = tile_bytes_of(kfmt);
  p.v_tile = tile_bytes_of(vfmt);
  p.k_norm_off = TQ_BLOCK_SIZE * row_index_bytes(kfmt);
  p.v_norm_off = TQ_BLOCK_SIZE * row_index_bytes(vfmt);
  const double mK = (double)D / kfmt->num_groups, mV = (double)D / vfmt->num_groups;
  p.score_mul = (float)((double)scale * 1.4426950408889634 / (sqrt((double)D) * sqrt(mK)));
  p.v_mul = (float)(1.0 / sqrt(mV));
  for (int jx = 0; jx < D; ++jx) {
    if (kfmt->signs[jx] < 0) p.k_signs[jx >> 5] |= 1u << (jx & 31);
    if (vfmt->signs[jx] < 0) p.v_signs[jx >> 5] |= 1u << (jx & 31);
    p.k_ch[jx] = kfmt->group_channels[jx];
  }
  // LUT halves: K's table in half 0; V shares it when bits and codebook agree
  const int kbits0 = kfmt->group_bits[0];
  p.half_kind[0] = kbits0;
  for (int i = 0; i < 16; ++i) p.half_cb[0][i] = kfmt->codebook[0][i];
  const int vbits = vfmt->group_bits[0];
  bool share = (kk == K4 || kk == KM43 || kk == K2) && vbits == kbits0;
  for (int i = 0; i < (1 << vbits) && share; ++i) share = vfmt->codebook[0][i] == kfmt->codebook[0][i];
  if (share) {
    p.v_half = 0;
    p.half_kind[1] = 0;
  } else {
    p.v_half = 1;
    p.half_kind[1] = vbits;
    for (int i = 0; i < 16; ++i) p.half_cb[1][i] = vfmt->codebook[0][i];
  }
  if (kk == KM43)
    for (int i = 0; i < 8; ++i) p.k3_cb[i] = kfmt->codebook[1][i];
  p.q_f32 = q_dtype == TQ_F32;
  p.out_f32 = out_dtype == TQ_F32;
  if (num_splits > 1) {
    p.part_o = static_cast<float*>(workspace);
    p.part_lse = p.part_o + (int64_t)num_seqs * num_q_heads * num_splits * D;
  }
  const unsigned grid = (unsigned)((items + 7) / 8 * 8);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
#define TQ_LAUNCH(DD, KKK, VVV)                                              \
  if (D == DD && kk == KKK && vk == VVV) launch_decode<DD, KKK, VVV>(p, grid, hs);
  TQ_LAUNCH(128, K4, V4) TQ_LAUNCH(128, K4, V2) TQ_LAUNCH(128, K2, V4) TQ_LAUNCH(128, K2, V2)
  TQ_LAUNCH(128, KM43, V4) TQ_LAUNCH(128, KM43, V2)
  TQ_LAUNCH(64, K4, V4) TQ_LAUNCH(64, K4, V2) TQ_LAUNCH(64, K2, V4) TQ_LAUNCH(64, K2, V2)
  TQ_LAUNCH(64, KM43, V4) TQ_LAUNCH(64, KM43, V2)
#undef TQ_LAUNCH
  st = launch_status("tq_decode_paged launch");
  if (st != TQ_OK || num_splits == 1) return st;
  MergeParams mp = {p.part_o, p.part_lse, out, lse, context_lens, num_seqs, num_q_heads, num_splits, D, p.C,
                    max_blocks_per_seq, p.out_f32};
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(num_seqs * num_q_heads)), dim3(64), 0, hs, mp);
  return launch_status("tq_decode_paged merge launch");
}
