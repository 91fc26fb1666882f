// Paged decode attention over packed, rotated, codebook-quantised K/V pages,
// plus the log-sum-exp merge of split partials.
//
// [D "Serving Route Design"]: block tables map logical to physical blocks;
// K rows are read inside the score computation and V rows are dequantised
// inside the accumulation; the workspace is bounded by the runtime shape.
// [D "System Invariants"]: production routes consume packed history (no dense
// K/V tensor is ever formed); unsupported formats raise.
//
// Work decomposition (balanced split-K).  Kv heads are taken in groups of
// HG adjacent heads (HG in 8, 4, 2, 1, chosen on the host).  The work is the
// list of (sequence, head group, logical block) units, sequence-major; a
// "segment" is the run of one (sequence, head group).  The grid is one
// persistent 16-wave workgroup per CU and workgroup w owns the contiguous
// range [w*R, (w+1)*R) of that list, so every workgroup gets the same number
// of blocks whatever the context lengths.  A workgroup walks the pieces of
// the segments its range covers; a segment that lies inside one range is
// finished there and written out directly, a segment cut by range
// boundaries leaves one partial (o, lse) per piece and q head in the
// workspace and the merge kernel combines them.  R is at least
// ceil(max_blocks / (P - 1)), so no segment has more than P pieces
// (P = num_splits, the workspace bound).
//
// Inside a piece, wave w serves kv head w % HG; the 16 / HG waves of a head
// take its blocks from an LDS counter (balanced however the SIMDs schedule
// them), each with its own online-softmax state, so the HG heads' tiles of
// a physical block (adjacent in the pool) are read at about the same time.
// The states are combined through LDS at the end of the piece.
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
// While block i is computed, the tiles of blocks i+1 and i+2 are in flight
// (three register buffers, loads never conditional).
// Codebook lookups use byte-indexed LDS tables replicated 32 times across
// the banks (one v_perm builds the address from a packed byte and the
// lane's copy); the tables sit at LDS offset 0 so the address needs no add.
// Epilogue: per (kv head, q head), combine the waves' states, inverse
// rotation once (Walsh-Hadamard across the wave, signs, 1/sqrt(d)).
#include <mutex>

#include "tq_internal.h"
#include "window_item.h"

namespace tq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));

constexpr int kWaves = 16;   // one workgroup per CU
constexpr int kThreads = kWaves * 64;
constexpr int kLutBytes = 65536;    // 256 entries x 256 B (two halves)
constexpr int kLut3Bytes = 4096;    // 64 entries x 16 copies x 4 B
constexpr int kBtCap = 2048;        // block-table entries of a piece staged in LDS
// Slot 0 of a row's partial lse holds this quiet NaN when the decode kernel
// has written the row's final output itself (nothing to merge).
constexpr uint32_t kDoneBits = 0x7FC0D0E5u;
constexpr float kLn2 = 0.6931471805599453f;

enum KKind { K4 = 0, K2 = 1, KM43 = 2, KM32 = 3 };
// K kinds with the QJL stage: the MSE kind plus this flag (sign bits after
// each row's MSE bytes, residual norms after the vector norms)
constexpr int KQ = 4;
enum VKind { V4 = 0, V2 = 1, VM43 = 2, VM32 = 3 };

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
  int64_t num_blocks;        // < 2^31
  int32_t S, Hq, Hkv, G, max_blocks, P;
  int32_t HG, NG;    // kv heads per workgroup group (1, 2, 4 or 8) and groups (Hkv / HG)
  // The G columns of a kv head are taken 8 at a time: column group cg holds
  // columns 8 cg .. 8 cg + 7 (CG groups, a power of two, 8 CG >= G).  A
  // (kv head, column group) pair is a virtual head; the HG kv heads of a
  // workgroup give VH = HG * CG <= 16 of them, each served by 16 / VH waves
  // that read the head's tiles (once from memory: the waves of the kv head
  // read each tile at about the same time).
  int32_t CG, VH;
  int32_t n_wg;      // grid size (persistent workgroups)
  int32_t seg_cost;  // work positions charged for starting a piece (see seg_span)
  float inv_G;       // 1 / G
  // Several queries per sequence (multi-query decode): the NQ * Gr (query, q
  // head) pairs of a kv head are its G = NQ * Gr <= 128 matrix-core columns
  // (column c: query c / Gr, q head c % Gr of the kv head); query i of a
  // sequence attends its first ctx - (NQ - 1 - i) cached tokens; q / out
  // rows are [sequence][query][q head].  NQ = 1, Gr = G for one query.
  int32_t NQ, Gr;
  int32_t rows_ps;   // q / out rows per sequence: NQ * Hq
  float inv_Gr;      // 1 / Gr
  int32_t k_tile, v_tile, k_norm_off, v_norm_off;
  uint32_t k_span, v_span;   // bytes of each pool (< 4 GiB)
  float score_mul;   // scale * log2(e) / (sqrt(D) * sqrt(m_K)), > 0
  const float* proj; // QJL: the projections S_g, fp32 [groups][m][m] (K kinds with KQ)
  // Dense window attended with the history (one query per sequence): bf16
  // rows [S][win_cap][Hkv][D], win_lens[s] valid; every row then goes
  // through the split merge, whose rows hold PS = P + 1 slots, the window's
  // result in slot P.  Without a window PS = P.
  const void* win_k;
  const void* win_v;
  const int32_t* win_lens;
  int32_t win_on, win_cap, PS;
  float win_scale_log2;   // softmax scale times log2(e)
  int32_t win_items;   // S * Hkv (sequence, kv head) window items, or 0
  float v_mul;       // 1 / sqrt(m_V), applied once in the epilogue
  uint32_t v_signs[4];
  uint32_t k_signs[4];
  uint16_t half_cb[2][16];   // codebook of the table in each LUT half
  int32_t half_kind[2];      // 0 none, 4 = nibble table, 2 = crumb table
  uint16_t k3_cb[8];         // 3-bit codebook of the mixed K low group
  uint8_t k_ch[128];
  uint8_t v_ch[128];         // V's listed channel order (two-group V formats)
  int32_t v_half;            // LUT half that V reads (its 4-bit or 2-bit group)
  int32_t q_f32, out_f32;
  int32_t q_bytes;           // size of q in bytes (< 2^31)
#ifdef TQ_PHASE_TRACE
  uint64_t* trace;           // per workgroup kTraceSlots timestamps (or null)
#endif
};

// Phase timestamps (built with TQ_PHASE_TRACE only): thread 0 of each
// workgroup records the 100 MHz real-time counter at kernel entry, when the
// plan is known, and per piece (up to 3) at its start, at the start and the
// end of its block loop and at the end of its epilogue; slot 14 at exit,
// slot 15 the number of pieces.
constexpr int kTraceSlots = 16;
#ifdef TQ_PHASE_TRACE
#define TQ_MARK(slot)                                                                       \
  do {                                                                                     \
    if (p.trace && threadIdx.x == 0 && (slot) < kTraceSlots)                               \
      p.trace[(int64_t)blockIdx.x * kTraceSlots + (slot)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define TQ_MARK_VALUE(slot, v)                                                       \
  do {                                                                               \
    if (p.trace && threadIdx.x == 0) p.trace[(int64_t)blockIdx.x * kTraceSlots + (slot)] = (v); \
  } while (0)
#else
#define TQ_MARK(slot) do {} while (0)
#define TQ_MARK_VALUE(slot, v) do {} while (0)
#endif


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


__device__ __forceinline__ float row_ror8(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true));
}

// Norm products.  K and V norms are applied as the f16 operand of a
// v_fma_mix (single rounding; under this library's build, fp16/fp64
// denormals on, the mix instructions take f16 subnormal operands and give
// subnormal fp16 results as they are: measured on gfx950, and pinned by
// the tiny-norm parity tests).  The fp16 P.V operand p * n_V carries a
// power-of-two factor 2^E per wave (E tracks the largest V norm seen, so
// that p * n_V * 2^E stays inside fp16's normal range whatever the scale of
// the rows; see the block loop).

// max of two floats known not to be NaN (no canonicalisation)
__device__ __forceinline__ float max_nn(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// One radix-2 stage of an unnormalised Walsh-Hadamard transform across
// lanes: the lane with bit K clear keeps the sum, the other the difference.
template <int K, int N>
__device__ __forceinline__ void wht_lanes(float (&x)[N], int lane) {
  const bool up = (lane & K) != 0;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float o = lane_xor<K>(x[e], lane);
    x[e] = up ? (o - x[e]) : (x[e] + o);
  }
}

// max over the lanes l, l^16, l^32, l^48 (gfx950 row and half swaps)
__device__ __forceinline__ float max_rows(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return max_nn(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}

__device__ __forceinline__ float half_at(uint2 w, int e) {
  const uint32_t d = (e >> 1) ? w.y : w.x;
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(d >> (16 * (e & 1))));
}

template <int D, int KK, int VK>
struct Cfg {
  static constexpr int R = D / 16;                       // dims per lane-row in P.V
  static constexpr int NQK = D / 32;                     // q.K MFMAs per block
  static constexpr int KB = KK & 3;                      // MSE kind of K
  static constexpr bool QJ = (KK & KQ) != 0;             // QJL stage on K
  static constexpr int KMSE = KB == K4 ? D / 2
                              : KB == K2 ? D / 4
                              : KB == KM43 ? (D / 2) * 4 / 8 + (D / 2) * 3 / 8
                                           : (D / 2) * 3 / 8 + (D / 2) * 2 / 8;
  static constexpr int KROW = KMSE + (QJ ? D / 8 : 0);   // K row stride: MSE bytes (+ sign bits)
  static constexpr int NGK = (KB == KM43 || KB == KM32) ? 2 : 1;   // K groups
  static constexpr int KRN = 16 * KROW + 32 * NGK;       // residual norms in a K tile (QJL)
  static constexpr int VROW = VK == V4 ? D / 2 : VK == V2 ? D / 4 : VK == VM43 ? (D / 2) * 7 / 8 : (D / 2) * 5 / 8;
  static constexpr int VLANE = VK == V4 ? D / 32 : D / 64;  // one-group V: bytes per lane per token
  static constexpr bool MIXED = NGK == 2;                 // two K groups
  // Two V groups: group g's octets (8 indices, b_g bytes) in runs of 4
  // tokens; lane (a, r) reads run (OCT a + r % OCT) of each group and holds
  // positions 8 (r % OCT) + (r / OCT) PPL + i (i < PPL) of its 4 tokens
  static constexpr bool MIXED_V = VK == VM43 || VK == VM32;
  static constexpr int VB0 = VK == VM43 ? 4 : 3, VB1 = VK == VM43 ? 3 : 2;   // bits of V groups 0, 1
  static constexpr int OCT = D / 16;                       // octets per V group (m / 8)
  static constexpr int PPL = D / 32;                       // positions per lane per V group (m / 16)
  static constexpr int VW0 = MIXED_V ? VB0 : 4;            // words of the lane's group-0 run (one group: v[4])
  static constexpr int VW = MIXED_V ? VB0 + VB1 : 4;       // V index words per lane per tile
  static constexpr int NVG = MIXED_V ? 2 : 1;              // V norm groups
  static constexpr bool PAIR3 = MIXED || MIXED_V;          // 3-bit pair table in use
  static constexpr int LDS_LUT = kLutBytes + (PAIR3 ? kLut3Bytes : 0);
  static constexpr int QV_FLOATS = NQK * 64 * 4;          // q.K B operands of one virtual head: NQK x 64 lanes x half8
  static constexpr int DS = D + 4;                        // wave-state row stride (floats)
  static constexpr int QX_FLOATS = kWaves * QV_FLOATS;           // operands of up to 16 virtual heads
  static constexpr int SX_FLOATS = kWaves * 8 * DS;              // wave states
  static constexpr int X_FLOATS = QX_FLOATS > SX_FLOATS ? QX_FLOATS : SX_FLOATS;
};

// Per-block raw loads of one wave.
template <int D, int KK, int VK>
struct Tile {
  uint32_t k[4];      // packed K bits of this lane (up to 16 B)
  uint32_t k_lo[2];   // mixed: low-group bits (aligned 8 B window)
  uint2 kn[2];        // K norms of the lane's 4 tokens, per group
  uint32_t v[Cfg<D, KK, VK>::VW];   // packed V bits of the lane's 4 tokens (raw words of its run(s))
  uint32_t sg;        // QJL: the dword holding the sign bytes of this lane's MFMAs (its K row)
  uint32_t gm;        // QJL: the dword holding the residual norm of its K row's token and group
  uint2 vn[Cfg<D, KK, VK>::NVG];    // V norms of the lane's 4 tokens, per group
};

// Buffer descriptor flags word for raw (untyped) loads: 32-bit data format.
constexpr int kBufFlags = 0x00020000;
// Cache policy of the page-tile loads: non-temporal (each tile is read once
// per call; measured 1.5-2% faster per decode call than the default policy).
constexpr int kTileAux = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, kBufFlags);
}

// One wave's loads of a block: buffer loads against the wave's pool
// descriptors (scalar base and range) with the lane's fixed offset as the
// vector offset and the block's byte offset plus compile-time constants as
// the scalar offset, so no vector address registers are live between issue
// and use (constants added to the vector offset would be hoisted out of the
// block loop into registers of their own).  V rows narrower than 4 B per
// lane are still loaded as a dword (the bytes past the lane's share stay
// inside the tile: the norm area follows the last row) so the loaded value
// needs no zero extension.
template <int D, int KK, int VK>
__device__ __forceinline__ void load_tile(Tile<D, KK, VK>& t, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                          uint32_t kb, uint32_t vb, uint32_t k_off, uint32_t klo_off,
                                          uint32_t n_off, uint32_t v_off, uint32_t v_off1, uint32_t sg_off,
                                          uint32_t gm_off) {
  using C = Cfg<D, KK, VK>;
  constexpr uint32_t KN = 16 * C::KROW, VN = 16 * C::VROW;   // norm areas follow the 16 rows
  if constexpr (C::KB == KM32) {   // the 2-bit group's bytes of this lane (aligned dword holding them)
    t.k[0] = __builtin_amdgcn_raw_buffer_load_b32(kr, k_off, kb, kTileAux);
  } else if constexpr (C::KB == K4 && D == 128) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(kr, k_off, kb, kTileAux);
    t.k[0] = x[0]; t.k[1] = x[1]; t.k[2] = x[2]; t.k[3] = x[3];
  } else if constexpr ((C::KB == K4 && D == 64) || (C::KB != K4 && D == 128)) {
    const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(kr, k_off, kb, kTileAux);
    t.k[0] = x[0]; t.k[1] = x[1];
  } else {
    t.k[0] = __builtin_amdgcn_raw_buffer_load_b32(kr, k_off, kb, kTileAux);
  }
  if constexpr (C::MIXED) {
    const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(kr, klo_off, kb, kTileAux);
    t.k_lo[0] = w[0];
    t.k_lo[1] = w[1];
  }
  {
    const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(kr, n_off, kb + KN, kTileAux);
    t.kn[0] = uint2{w[0], w[1]};
  }
  if constexpr (C::MIXED) {
    const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(kr, n_off, kb + KN + 32u, kTileAux);
    t.kn[1] = uint2{w[0], w[1]};
  }
  if constexpr (C::QJ) {
    t.sg = __builtin_amdgcn_raw_buffer_load_b32(kr, sg_off, kb, kTileAux);
    t.gm = __builtin_amdgcn_raw_buffer_load_b32(kr, gm_off, kb, kTileAux);
  }
  // lane-major V plane: the lane's run holds its bytes of tokens a, a+4, a+8,
  // a+12 back to back (raw words; compute() picks each token's bytes); two
  // groups: the lane's run of each group's sub-plane (4 b_g bytes)
  if constexpr (C::MIXED_V) {
    auto run = [&](uint32_t* dst, int words, uint32_t off) {
      if (words == 4) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(vr, off, vb, kTileAux);
        dst[0] = x[0]; dst[1] = x[1]; dst[2] = x[2]; dst[3] = x[3];
      } else if (words == 3) {
        const u32x3_t x = __builtin_amdgcn_raw_buffer_load_b96(vr, off, vb, kTileAux);
        dst[0] = x[0]; dst[1] = x[1]; dst[2] = x[2];
      } else {
        const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(vr, off, vb, kTileAux);
        dst[0] = x[0]; dst[1] = x[1];
      }
    };
    run(t.v, C::VB0, v_off);
    run(t.v + C::VB0, C::VB1, v_off1);
  } else if constexpr (C::VLANE == 4) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(vr, v_off, vb, kTileAux);
    t.v[0] = x[0]; t.v[1] = x[1]; t.v[2] = x[2]; t.v[3] = x[3];
  } else if constexpr (C::VLANE == 2) {
    const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(vr, v_off, vb, kTileAux);
    t.v[0] = x[0]; t.v[1] = x[1];
  } else {
    t.v[0] = __builtin_amdgcn_raw_buffer_load_b32(vr, v_off, vb, kTileAux);
  }
  {
    const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(vr, n_off, vb + VN, kTileAux);
    t.vn[0] = uint2{w[0], w[1]};
  }
  if constexpr (C::MIXED_V) {
    const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(vr, n_off, vb + VN + 32u, kTileAux);
    t.vn[1] = uint2{w[0], w[1]};
  }
}

// Uniform read of a value the kernel never writes, through the scalar cache
// (a constant-address-space load), so that waiting for it does not order it
// with the vector loads in flight.
__device__ __forceinline__ int scalar_ld(const int32_t* ptr, int idx) {
  return ((const __attribute__((address_space(4))) int32_t*)ptr)[idx];
}

__device__ __forceinline__ int clamp_ctx(int c, int cap) { return c < 0 ? 0 : (c > cap ? cap : c); }

// The lane index, recomputed where it is called: values derived from it
// are then not kept live across the block loop (which has no registers to
// spare) but rebuilt where they are needed.
__device__ __forceinline__ int fresh_lane() {
  int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(l));
  return l;
}

// A value known to be the same in every lane, moved to a scalar register so
// that everything derived from it (addresses above all) stays scalar.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int K>
__device__ __forceinline__ int lane_xor_i(int v, int lane) {
  return __float_as_int(lane_xor<K>(__int_as_float(v), lane));
}

// Wave-wide sum (every lane gets it).
__device__ __forceinline__ int wave_sum(int v, int lane) {
  v += lane_xor_i<32>(v, lane);
  v += lane_xor_i<16>(v, lane);
  v += lane_xor_i<8>(v, lane);
  v += lane_xor_i<4>(v, lane);
  v += lane_xor_i<2>(v, lane);
  v += lane_xor_i<1>(v, lane);
  return v;
}

// Wave-wide inclusive prefix sum over lanes: shifts within each 16-lane row
// (DPP row_shr 1, 2, 4, 8 give lane i the value of lane i - k), then the
// row totals are carried up with the row broadcasts (lane 15 of a row to the
// next row, lane 31 to the upper half).
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
  const int r = lane & 15;
  int t = __builtin_amdgcn_mov_dpp(x, 0x111, 0xF, 0xF, true);
  if (r >= 1) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x112, 0xF, 0xF, true);
  if (r >= 2) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x114, 0xF, 0xF, true);
  if (r >= 4) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x118, 0xF, 0xF, true);
  if (r >= 8) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x142, 0xF, 0xF, true);   // row_bcast 15
  if (lane & 16) x += t;
  t = __builtin_amdgcn_mov_dpp(x, 0x143, 0xF, 0xF, true);   // row_bcast 31
  if (lane & 32) x += t;
  return x;
}

// Context lengths, clamped to [0, 16 max_blocks]: cl0 holds sequence `lane`
// (sequences 0-63, read once per kernel, kept in LDS as s_cl); later
// sequences are read on use.
__device__ __forceinline__ int seq_len(const DecodeParams& p, const int* s_cl, int s) {
  if (s < 64) return __builtin_amdgcn_readfirstlane(s_cl[s]);
  return clamp_ctx(scalar_ld(p.context_lens, s), p.max_blocks * 16);
}
__device__ __forceinline__ int lane_len(const DecodeParams& p, int cl0, int base, int lane) {
  const int sq = base + lane;
  if (sq >= p.S) return 0;
  return base == 0 ? cl0 : clamp_ctx(p.context_lens[sq], p.max_blocks * 16);
}

// Work positions: a (sequence, kv-head group) segment of nb > 0 blocks spans
// seg_cost + nb positions, a fixed charge for starting a piece (its set-up
// and epilogue) followed by one position per block, so that a workgroup
// range that covers a segment start gets fewer blocks.  Sequences with no
// block have no segment.
__device__ __forceinline__ int seg_span(const DecodeParams& p, int nb) { return nb > 0 ? nb + p.seg_cost : 0; }

// Wave-wide: total work W = NG * sum of segment spans (all lanes get it).
__device__ int total_work(const DecodeParams& p, int cl0, int lane) {
  int tot = 0;
  for (int base = 0; base < p.S; base += 64)
    tot += uni(wave_sum(seg_span(p, (lane_len(p, cl0, base, lane) + 15) >> 4), lane));
  return tot * p.NG;
}

// Wave-wide: the segment that contains work position pos (pos < W): its
// sequence, kv-head group, block count and the offset of pos in its span.
__device__ void locate(const DecodeParams& p, int cl0, int lane, int pos, int& s, int& grp, int& off, int& nb_s) {
  int before = 0;
  s = -1;
  grp = off = nb_s = 0;
  for (int base = 0; base < p.S && s < 0; base += 64) {
    const int cnt = seg_span(p, (lane_len(p, cl0, base, lane) + 15) >> 4) * p.NG;
    const int incl = wave_incl_scan(cnt, lane);
    const int excl = incl - cnt;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(base + lane < p.S && pos >= before + excl && pos < before + incl);
    if (hit) {
      const int src = uni(__builtin_ctzll(hit));
      s = base + src;
      const int r = pos - before - __builtin_amdgcn_readlane(excl, src);
      const int span = __builtin_amdgcn_readlane(cnt, src) / p.NG;
      nb_s = span - p.seg_cost;
      grp = r / span;
      off = r % span;
    }
    before += __builtin_amdgcn_readlane(incl, 63);
  }
}

// Wave-wide: the first segment start at or after work position x (W if none).
__device__ int snap_to_segment(const DecodeParams& p, int cl0, int lane, int x, int W) {
  if (x >= W) return W;
  int s, grp, off, nb;
  locate(p, cl0, lane, x, s, grp, off, nb);
  return off == 0 ? x : x - off + seg_span(p, nb);
}

// Positions per workgroup range: an even share of the work and, when
// segments may be split (P > 1), at least ceil(max_blocks / (P - 1)) so that
// the blocks of no segment meet more than P ranges.  With P == 1 the range boundaries are
// moved to segment starts (see snap_to_segment) and no segment is split.
__device__ __forceinline__ int range_len(int W, int n_wg, int max_blocks, int P) {
  int R = (W + n_wg - 1) / n_wg;
  if (R < 1) R = 1;
  if (P == 1) return R;
  const int need = (max_blocks + P - 2) / (P - 1);
  return R > need ? R : need;
}

// Waves -> (virtual head of the group, part).  The 16 waves sit on the 4
// SIMDs as wave % 4, and on a SIMD older waves (lower index) issue first.
// With 8 heads of 2 parts, head h % 4 + 4 b is served by the waves of ranks
// {0, 3} (b = 0) or {1, 2} (b = 1) on SIMD h % 4, so that every head gets
// the same share of issue slots; otherwise head h has parts h + VH q.
__device__ __forceinline__ int head_of_wave(int wave, int VH) {
  if (VH == 8) {
    const int r = wave >> 2;
    return (wave & 3) | (((r ^ (r >> 1)) & 1) << 2);
  }
  return wave % VH;
}
__device__ __forceinline__ int part_of_wave(int wave, int VH) { return VH == 8 ? wave >> 3 : wave / VH; }
__device__ __forceinline__ int wave_of_part(int h, int q, int VH) {
  if (VH == 8) return 4 * (q ? ((h & 4) ? 2 : 3) : ((h & 4) ? 1 : 0)) + (h & 3);
  return h + VH * q;
}

// Workgroup barrier that orders LDS accesses only: the waves' global loads
// (the first page tiles) stay in flight across it, where __syncthreads would
// wait for every outstanding load.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup LDS.  The tables come first so that every table address
// (< 64 KB) fits the immediate offset of the LDS read.
template <int D, int KK, int VK>
struct Smem {
  using C = Cfg<D, KK, VK>;
  uint8_t lut[C::LDS_LUT];
  // per virtual head: q.K operands (NQK x 64 lanes x half8); after the
  // block loop the same bytes hold the wave states
  float xbuf[C::X_FLOATS];
  float s_ml[kWaves * 16];   // per wave: running max and sum of each column
  uint32_t s_par[64];
  uint32_t s_vch[32];        // V's listed channel order, 4 per word (two-group V)
  int s_qexp[8 * kWaves];    // [virtual head][column]
  float s_rq[64];            // QJL: [virtual head][column] weight of the sketch sum against the q.K sum
  int s_next[kWaves];        // per virtual head: next free piece block
  int s_bt[kBtCap];          // block-table entries of the piece's first kBtCap blocks
  int s_cl[64];              // clamped context lengths of sequences 0-63
  int s_plan[10];            // work split: R, range start and end, first segment, window items
};

template <int D, int KK, int VK>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p) {
  using C = Cfg<D, KK, VK>;
  constexpr int R4 = 4 * C::R;   // output dims per lane
  constexpr int NQK = C::NQK;
  __shared__ __attribute__((aligned(16))) Smem<D, KK, VK> sm;
  uint8_t* const lds = sm.lut;
  float* const xbuf = sm.xbuf;
  float* const s_ml = sm.s_ml;
  uint32_t* const s_par = sm.s_par;
  uint32_t* const s_vch = sm.s_vch;
  int* const s_qexp = sm.s_qexp;
  float* const s_rq = sm.s_rq;
  int* const s_next = sm.s_next;
  int* const s_bt = sm.s_bt;
  int* const s_cl = sm.s_cl;
  int* const s_plan = sm.s_plan;

  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6);
  const int lane = tid & 63;
  TQ_MARK(0);
  // ---- wave 0 plans: it alone reads the context lengths and splits the
  // work, and publishes its results in LDS; wave 1 meanwhile spreads the
  // small per-call tables (kernel arguments read at compile-time offsets
  // only, then spread over lanes by lane selects; lane-indexed reads of the
  // argument block would be slow per-lane vector loads)
  if (wave == 0) {
    // Touch every 64-byte line of the argument block at once: the first read
    // of a line misses the scalar cache, and the fields are read at many
    // points of the set-up, which would otherwise wait for a miss each.
    {
      const __attribute__((address_space(4))) uint32_t* ka =
          (const __attribute__((address_space(4))) uint32_t*)__builtin_amdgcn_kernarg_segment_ptr();
      constexpr int kLines = (int)((sizeof(DecodeParams) + 63) / 64);
      uint32_t kw[kLines];
#pragma unroll
      for (int i = 0; i < kLines; ++i) kw[i] = ka[16 * i];   // all issued before the first use waits
#pragma unroll
      for (int i = 0; i < kLines; ++i) asm volatile("" ::"s"(kw[i]));
    }
    // context length of sequence `lane` (lanes past the last sequence read 0
    // through the descriptor's range check)
    const int cl_raw = (int)__builtin_amdgcn_raw_buffer_load_b32(
        tile_rsrc(reinterpret_cast<const uint8_t*>(p.context_lens), 4 * p.S), (uint32_t)(4 * lane), 0, 0);
    const int cap = p.max_blocks * 16;
    const int cl0 = clamp_ctx(cl_raw, cap);
    s_cl[lane] = cl0;
    // context lengths outside [0, 16 * max_blocks] are reported (first
    // workgroup) and clamped
    if (blockIdx.x == 0 && lane < p.S && (cl_raw < 0 || cl_raw > cap)) record_error(p.dev_err, TQ_ERR_INDEX, -1 - lane);
    const int W = total_work(p, cl0, lane);
    const int R = range_len(W, p.n_wg, p.max_blocks, p.P);
    int r0 = blockIdx.x * R;
    int r1 = (r0 + R < W) ? r0 + R : W;
    // window items: an even share for every workgroup, run after its pieces
    // (a workgroup given only window items streams them latency-bound, far
    // slower than the pieces' rate, so they are not traded against pieces)
    // (32-bit: win_items * n_wg < 2^32 by the host's work bound; no
    // division at all without a window)
    const int i0 = p.win_items ? (int)(blockIdx.x * (uint32_t)p.win_items / (uint32_t)p.n_wg) : 0;
    const int i1 = p.win_items ? (int)((blockIdx.x + 1) * (uint32_t)p.win_items / (uint32_t)p.n_wg) : 0;
    if (p.P == 1) {   // whole segments only: there is no workspace for partials
      r0 = snap_to_segment(p, cl0, lane, r0, W);
      r1 = snap_to_segment(p, cl0, lane, r1, W);
    }
    int s0 = 0, grp0 = 0, off0 = 0, nb0 = 0;
    if (r0 < r1) locate(p, cl0, lane, r0, s0, grp0, off0, nb0);
    if (lane == 0) {
      s_plan[0] = R; s_plan[1] = r0; s_plan[2] = r1; s_plan[3] = s0;
      s_plan[4] = grp0; s_plan[5] = off0; s_plan[6] = nb0;
      s_plan[7] = i0; s_plan[8] = i1;
    }
  } else if (wave == 1) {
    uint32_t x = 0;
    auto put = [&](uint32_t v, int i, uint32_t cur) -> uint32_t { return lane == i ? v : cur; };
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x = put((uint32_t)p.half_cb[0][2 * i] | ((uint32_t)p.half_cb[0][2 * i + 1] << 16), i, x);
      x = put((uint32_t)p.half_cb[1][2 * i] | ((uint32_t)p.half_cb[1][2 * i + 1] << 16), 8 + i, x);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x = put((uint32_t)p.k3_cb[2 * i] | ((uint32_t)p.k3_cb[2 * i + 1] << 16), 16 + i, x);
      x = put(p.k_signs[i], 20 + i, x);
      x = put(p.v_signs[i], 24 + i, x);
    }
    if constexpr (C::MIXED) {
#pragma unroll
      for (int i = 0; i < 32; ++i)
        x = put((uint32_t)p.k_ch[4 * i] | ((uint32_t)p.k_ch[4 * i + 1] << 8) | ((uint32_t)p.k_ch[4 * i + 2] << 16) |
                    ((uint32_t)p.k_ch[4 * i + 3] << 24),
                32 + i, x);
    }
    s_par[lane] = x;
    if constexpr (C::MIXED_V) {
      uint32_t y = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i)
        y = put((uint32_t)p.v_ch[4 * i] | ((uint32_t)p.v_ch[4 * i + 1] << 8) | ((uint32_t)p.v_ch[4 * i + 2] << 16) |
                    ((uint32_t)p.v_ch[4 * i + 3] << 24),
                i, y);
      if (lane < 32) s_vch[lane] = y;
    }
  }
  __syncthreads();   // plan, lengths and s_par written
  TQ_MARK(1);

  // ---- the plan (uniform values)
  const int R = uni(s_plan[0]);
  const int r0 = uni(s_plan[1]), r1 = uni(s_plan[2]);

  // sequences with no cached token: out = 0, lse = -inf (first workgroup;
  // lengths of sequences past the first 64 are reported here)
  if (blockIdx.x == 0) {
    const int cap = p.max_blocks * 16;
    for (int s = wave; s < p.S; s += kWaves) {
      int c;
      if (s < 64) {
        c = uni(s_cl[s]);
      } else {
        c = p.context_lens[s];
        if (lane == 0 && (c < 0 || c > cap)) record_error(p.dev_err, TQ_ERR_INDEX, -1 - s);
        c = clamp_ctx(c, cap);
      }
      if (c == 0 && p.win_on) {   // the window alone: empty history slots for the merge
        for (int h = lane; h < p.rows_ps * p.P; h += 64)
          p.part_lse[((int64_t)s * p.rows_ps + h / p.P) * p.PS + h % p.P] = -INFINITY;
      } else if (c == 0) {
        for (int idx = lane; idx < p.rows_ps * D; idx += 64) {
          const int64_t off = (int64_t)s * p.rows_ps * D + idx;
          if (p.out_f32) static_cast<float*>(p.out)[off] = 0.f;
          else static_cast<uint16_t*>(p.out)[off] = 0;
        }
        if (p.lse)
          for (int h = lane; h < p.rows_ps; h += 64) p.lse[(int64_t)s * p.rows_ps + h] = -INFINITY;
        if (p.P > 1)   // tell the merge that these rows are final
          for (int h = lane; h < p.rows_ps; h += 64) p.part_lse[((int64_t)s * p.rows_ps + h) * p.PS] = __uint_as_float(kDoneBits);
      }
    }
  }
  // dense window: the workgroup's (sequence, kv head) items after its
  // pieces, in the LDS of the tables and operands (free by then), each
  // result to slot P of its rows
  auto window_items = [&]() {
    const int i0 = uni(s_plan[7]), i1 = uni(s_plan[8]);
    if (i0 >= i1) return;
    using W = WinItemCfg<D, 16, kThreads, 128>;
    static_assert(W::BYTES <= (int)(sizeof(sm.lut) + sizeof(sm.xbuf)), "window item larger than its LDS");
    WindowParams wp = {};
    wp.q = p.q; wp.k = p.win_k; wp.v = p.win_v; wp.lens = p.win_lens;
    wp.dev_err = p.dev_err;
    wp.S = p.S; wp.Hq = p.Hq; wp.Hkv = p.Hkv; wp.G = p.Gr; wp.cap = p.win_cap;
    wp.scale_log2 = p.win_scale_log2;
    wp.q_f32 = p.q_f32;
    WinSink sink;
    sink.part_o = p.part_o;
    sink.part_lse = p.part_lse;
    sink.PS = p.PS;
    sink.slot = p.P;
    __syncthreads();   // the workgroup is done with the LDS of its pieces
    window_items_bf16<D, 16, kThreads, 128, 1>(wp, sink, i0, i1, sm.lut, tid);
  };
  int n_done = 0;   // pieces this workgroup has run (phase trace)
  if (r0 < r1) {  // uniform across the workgroup; else the window items only
    auto cb_half = [&](int h, int i) -> uint32_t { return (s_par[8 * h + (i >> 1)] >> (16 * (i & 1))) & 0xFFFFu; };

    // LDS tables: byte-indexed, two halves of 128 B per entry, built once
    // (while the first piece's block-table, q and tile loads are in flight).
    // Thread -> 16 B chunk (16 e + lane & 15) of entry e = 16 e_hi + e_lo:
    // lane & 15 walks the 256 B of an entry (8 chunks per half), so each
    // store instruction writes 1 KB contiguous; e_lo is fixed per lane,
    // e_hi = (wave >> 2) + 4 it.
    auto build_tables = [&]() {
      const int h = (lane >> 3) & 1;
      const int e_lo = (lane >> 4) | ((wave & 3) << 2);
      const int wh = wave >> 2;
      const uint32_t sh = (uint32_t)(wh & 1) * 16u;
      const int kind0 = uni(p.half_kind[0]), kind1 = uni(p.half_kind[1]);   // scalar reads
      const int kind = h ? kind1 : kind0;
      const uint4 r03 = *reinterpret_cast<const uint4*>(s_par + 8 * h);
      const uint4 r47 = *reinterpret_cast<const uint4*>(s_par + 8 * h + 4);
      const uint32_t cw[8] = {r03.x, r03.y, r03.z, r03.w, r47.x, r47.y, r47.z, r47.w};
      const uint32_t lo_n = cb_half(h, e_lo);
      const uint32_t ev = cb_half(h, e_lo & 3) | (cb_half(h, e_lo >> 2) << 16);
      const uint32_t c2 = (((wh >> 1) ? cw[1] : cw[0]) >> sh) & 0xFFFFu;   // cb[e_hi & 3] = cb[wh]
      uint4* dst = reinterpret_cast<uint4*>(lds) + (lane & 15) + 16 * e_lo + 256 * wh;
  #pragma unroll
      for (int it = 0; it < 4; ++it) {
        // nibble table: (cb[e & 15], cb[e >> 4]);
        // crumb table: (cb[e & 3], cb[(e >> 2) & 3]), (cb[(e >> 4) & 3], cb[e >> 6])
        const uint32_t hiw = (wh >> 1) ? cw[2 * it + 1] : cw[2 * it];
        const uint32_t v4 = lo_n | (((hiw >> sh) & 0xFFFFu) << 16);
        const uint32_t c3 = (cw[it >> 1] >> (16 * (it & 1))) & 0xFFFFu;
        const uint32_t od = c2 | (c3 << 16);
        const uint32_t x0 = kind == 4 ? v4 : (kind == 2 ? ev : 0u);
        const uint32_t x1 = kind == 4 ? v4 : (kind == 2 ? od : 0u);
        dst[1024 * it] = uint4{x0, x1, x0, x1};
      }
      if constexpr (C::PAIR3) {
        for (int c = tid; c < kLut3Bytes / 16; c += kThreads) {
          const int e = c >> 2;
          const uint32_t lo = (s_par[16 + ((e & 7) >> 1)] >> (16 * (e & 1))) & 0xFFFFu;
          const uint32_t hi = (s_par[16 + ((e >> 3) >> 1)] >> (16 * ((e >> 3) & 1))) & 0xFFFFu;
          const uint32_t v = lo | (hi << 16);
          reinterpret_cast<uint4*>(lds + kLutBytes)[c] = uint4{v, v, v, v};
        }
      }
    };

    // ---- per-lane roles
    const int j = lane & 15;          // MFMA column: q head j & 7, high (j < 8) or low part
    const int a = lane >> 4;          // token group: tokens a, a+4, a+8, a+12 of a block
    const int gq = j & 7;
    const bool lo_part = j >= 8;
    const uint32_t off4_k = (uint32_t)(lane & 31) * 4u;                      // K nibble table, half 0
    const uint32_t off2_k = (uint32_t)(lane & 15) * 8u;                      // K crumb table, half 0
    const uint32_t off_v4 = (uint32_t)p.v_half * 128u + (uint32_t)(lane & 31) * 4u;
    const uint32_t off_v2 = (uint32_t)p.v_half * 128u + (uint32_t)(lane & 15) * 8u;
    const uint32_t off3 = (uint32_t)kLutBytes + (uint32_t)(lane & 15) * 4u;
    const int tokK = (j >> 2) + 4 * (j & 3);   // token of this lane's K row: sigma(j)
    // per-lane byte offsets inside a K / V tile: k_off the lane's bytes of the
    // one group (K4, K2) or of the 4-bit group (4+3), or the aligned dword that
    // holds its bytes of the 2-bit group (3+2); klo_off the aligned 8-B window
    // that holds its bytes of the 3-bit group (two-group formats)
    constexpr int KLANE = C::KB == K4 ? D / 8 : D / 16;
    constexpr int G3_AT = C::KB == KM32 ? 0 : D / 4;   // first byte of the 3-bit group in a row
    const uint32_t k_off = C::KB == KM32 ? (uint32_t)((tokK * C::KROW + 3 * D / 16 + (D / 32) * a) & ~3)
                                      : (uint32_t)(tokK * C::KROW + KLANE * a);
    const uint32_t klo_off = (uint32_t)((tokK * C::KROW + G3_AT + (3 * D / 64) * a) & ~3);
    const uint32_t n_off = (uint32_t)(8 * a);   // this lane's 4 norms, after the tile's norm offset
    // QJL: the aligned dword holding the sign bytes NQK a .. NQK a + NQK - 1 of
    // its K row (sketch output 32 a + 8 t + e of MFMA t is bit e of byte 4 a +
    // t; d = 64: 16 a + 8 t + e, byte 2 a + t), and the one holding the
    // residual norm of the row's token (norm slot j) for the group of those
    // outputs, (a NGK) / 4
    const uint32_t sg_off = (uint32_t)(tokK * C::KROW + C::KMSE + ((NQK * a) & ~3));
    const uint32_t gm_off = (uint32_t)(C::KRN + 2 * (16 * ((a * C::NGK) >> 2) + (j & ~1)));
    // this lane's run of the V plane (two groups: its run of each sub-plane,
    // group 1's sub-plane after group 0's 16 (D / 2) VB0 / 8 bytes)
    const int vrun = C::OCT * (lane >> 4) + (lane & 15) % C::OCT;
    const uint32_t v_off = C::MIXED_V ? (uint32_t)(vrun * 4 * C::VB0) : (uint32_t)(lane * 4 * C::VLANE);
    const uint32_t v_off1 = (uint32_t)(16 * ((D / 2) * C::VB0 / 8) + vrun * 4 * C::VB1);
    const int64_t k_blk_stride = (int64_t)p.Hkv * p.k_tile;
    const int64_t v_blk_stride = (int64_t)p.Hkv * p.v_tile;
    const int cap = p.max_blocks * 16;
    // wave -> (virtual head of the group, part): the NPW waves of a virtual
    // head share its blocks; virtual head vh is column group cg of kv head hl
    const int HG = p.HG, CG = p.CG, VH = p.VH;
    const int NPW = kWaves / VH;
    const int vh = uni(head_of_wave(wave, VH));
    const int part = uni(part_of_wave(wave, VH));
    const int hl = uni(vh / CG);
    const int cg = uni(vh - hl * CG);
    half8_t* const qv_all = reinterpret_cast<half8_t*>(xbuf);            // [vh][t][lane]
    float* const slots = xbuf;                                           // [wave][g] rows of DS floats

    // ---- walk the pieces of this workgroup's range
    int s = uni(s_plan[3]), grp = uni(s_plan[4]), off = uni(s_plan[5]), nb_s = uni(s_plan[6]);
    int pos = r0;
    bool first = true;
    bool tables_built = false;
    while (pos < r1) {
      const int vb0 = pos - off + p.seg_cost;   // position of the segment's block 0
      const int b0 = off > p.seg_cost ? off - p.seg_cost : 0;
      const int b1 = (r1 - vb0 < nb_s) ? r1 - vb0 : nb_s;
      if (b1 > b0) {   // the range holds blocks of this segment
      // one piece: the final output is written here (always so when P == 1)
      // with a window every row is merged: a whole segment writes slot 0
      const bool whole = !p.win_on && (p.P == 1 || (vb0 / R) == ((vb0 + nb_s - 1) / R));
      const int piece = p.P == 1 ? 0 : (int)blockIdx.x - vb0 / R;
      const int n_pieces = p.P == 1 ? 1 : (vb0 + nb_s - 1) / R - vb0 / R + 1;
        const int ctx = seq_len(p, s_cl, s);
        // causal lengths: the sequence's last NQ cached tokens are the queries'
        // own, query i sees ctx - (NQ - 1 - i) of them; ctx_all is what every
        // query sees, ctx_col this lane's column's (columns past G: ctx)
        const int ctx_all = ctx - (p.NQ - 1);
        const int qi_col = (int)(((float)(8 * cg + gq) + 0.5f) * p.inv_Gr);
        const int ctx_col = qi_col < p.NQ ? ctx - (p.NQ - 1 - qi_col) : ctx;
        const int kvh = grp * HG + hl;   // this wave's kv head
        const uint8_t* k_head = p.k_pages + (int64_t)kvh * p.k_tile;
        const uint8_t* v_head = p.v_pages + (int64_t)kvh * p.v_tile;
        const int32_t* bt_row = p.block_tables + (int64_t)s * p.max_blocks;

        if (!first) __syncthreads();   // the previous piece's states have been read
        first = false;
        TQ_MARK(2 + 4 * n_done);

        // -------- blocks of the piece are handed out per kv head: part q of a
        // head starts with piece blocks q, q + NPW and q + 2 NPW, then takes the
        // next free index from the head's LDS counter, so parts that run ahead
        // take more blocks and all finish together.  The HG heads of the group
        // read the HG adjacent tiles of each physical block at about the same
        // time.  The piece's block-table entries are staged in LDS (the first
        // kBtCap of them; later ones are read from memory), so a block costs
        // index (LDS atomic) -> entry (LDS read) -> tile loads; while a tile is
        // computed the next two tiles are in flight.
        const int n = b1 - b0;   // blocks of the piece, >= 1
        if (tid < kWaves) s_next[tid] = 3 * NPW;
        const __amdgpu_buffer_rsrc_t btr = tile_rsrc(reinterpret_cast<const uint8_t*>(bt_row), 4 * p.max_blocks);
        auto bt_load = [&](int idx) -> int {   // entry of piece block idx (block b0 when idx >= n)
          return (int)__builtin_amdgcn_raw_buffer_load_b32(btr, 0u, 4 * (b0 + (idx < n ? idx : 0)), 0);
        };
        constexpr int NBT = kBtCap / kThreads;
        int btv[NBT];
  #pragma unroll
        for (int i = 0; i < NBT; ++i) {
          const int e = tid + kThreads * i;
          btv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(btr, (uint32_t)(4 * (e < n ? e : 0)), 4 * b0, 0);
        }
        constexpr int PER = D / 8;              // q channels per lane in the rotation, 8 lanes per column
        const int ln = fresh_lane();
        const int g8 = ln >> 3, l8 = ln & 7;
        const int colq = 8 * cg + g8;           // this lane's column in the rotation
        const bool q_live = colq < p.G;
        // raw q words of this lane's PER channels (bf16: two per word, the upper
        // half of qw unused); one load shape for both dtypes, bytes past the q
        // tensor read as zero through the descriptor's range check
        uint32_t qw[PER];
        {   // issued by every wave so that all paths carry the same loads and
            // later waits count exactly; parts > 0 discard them and read
            // through an empty range (no memory access): on a long context
            // hundreds of workgroups read the same few q rows at once
          const int esz = p.q_f32 ? 4 : 2;
          const int head0 = uni((int)(((int64_t)s * p.rows_ps + kvh * p.Gr) * D * esz));   // query 0, first q head
          int qrow = 0;   // this lane's (query, q head) column: rows past head0
          if (q_live) {
            const int qi = (int)(((float)colq + 0.5f) * p.inv_Gr);
            qrow = qi * p.Hq + (colq - qi * p.Gr);
          }
          const uint32_t lane_off = (uint32_t)((qrow * D + l8 * PER) * esz);
          const __amdgpu_buffer_rsrc_t qr = tile_rsrc(static_cast<const uint8_t*>(p.q), part == 0 ? p.q_bytes : 0);
  #pragma unroll
          for (int i = 0; i < PER / 4; ++i) {
            const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(qr, lane_off + 16 * i, head0, 0);
            qw[4 * i] = t[0]; qw[4 * i + 1] = t[1]; qw[4 * i + 2] = t[2]; qw[4 * i + 3] = t[3];
          }
        }
        // QJL: wave w computes output tile ot_w = w % (D / 16) of the projected
        // rows (16 outputs) for virtual heads w / (D / 16), + 16 / (D / 16), ...;
        // its S values (the same for all of them) are requested here, before
        // the tiles, so that waiting for them does not wait for the tiles
        constexpr int QOT = D / 16, QM = D / C::NGK, QKC = QM / 32;
        const int ot_w = wave % QOT;
        float4 spf[C::QJ ? 2 * QKC : 1];
        if constexpr (C::QJ) {
          const int lp = fresh_lane();
          const float* srow = p.proj + ((int64_t)(16 * ot_w + (lp & 15)) * QM + 8 * (lp >> 4));
  #pragma unroll
          for (int kc = 0; kc < QKC; ++kc) {
            spf[2 * kc] = *reinterpret_cast<const float4*>(srow + 32 * kc);
            spf[2 * kc + 1] = *reinterpret_cast<const float4*>(srow + 32 * kc + 4);
          }
        }
        int idx_c = part, idx_1 = part + NPW, idx_2 = part + 2 * NPW;
        const int v0 = bt_load(idx_c);
        const int v1 = bt_load(idx_1);
        if (!tables_built) {   // while the loads above are in flight
          build_tables();
          tables_built = true;
        }

        // -------- block-table entry -> scalar byte offsets of the block's tiles
        // in the pools (whose bytes, less than 4 GiB each, one descriptor per
        // wave covers); entries outside the pool are reported and their block
        // skipped (read as block 0)
        const __amdgpu_buffer_rsrc_t kt = tile_rsrc(k_head, (int)(p.k_span - (uint32_t)kvh * (uint32_t)p.k_tile));
        const __amdgpu_buffer_rsrc_t vt = tile_rsrc(v_head, (int)(p.v_span - (uint32_t)kvh * (uint32_t)p.v_tile));
        uint32_t kb, vb;
        auto entry = [&](int v, int idx, bool& ok) {
          const uint32_t raw = (uint32_t)__builtin_amdgcn_readfirstlane(v);
          const bool live = idx < n;
          const bool bad = live && raw >= (uint32_t)p.num_blocks;
          if (bad && lane == 0) record_error(p.dev_err, TQ_ERR_INDEX, s * p.max_blocks + b0 + idx);
          const uint32_t ph = (uint32_t)uni(bad ? 0 : (int)raw);
          ok = live && !bad;
          kb = ph * (uint32_t)k_blk_stride;
          vb = ph * (uint32_t)v_blk_stride;
        };
        auto bt_at = [&](int idx) -> int {   // entry value of piece block idx (any lane)
          if (idx >= n) return 0;
          if (idx < kBtCap) return s_bt[idx];
          const int v = bt_load(idx);        // long piece: read from memory (latency exposed)
          return __builtin_amdgcn_readfirstlane(v);
        };
        auto grab = [&]() -> int {   // next free piece block of this head (valid in lane 0)
          int g = 0;
          if (lane == 0) g = atomicAdd(&s_next[vh], 1);
          return g;
        };
        Tile<D, KK, VK> A, B, C3;
        bool ok_c, ok_1;
        // the first two tiles go out now, so that their latency overlaps the
        // q rotation (and the QJL projection): the barriers up to the block
        // loop order LDS accesses only, so the tile loads stay in flight
        auto first_tiles = [&]() {
          entry(v0, idx_c, ok_c);
          load_tile<D, KK, VK>(A, kt, vt, kb, vb, k_off, klo_off, n_off, v_off, v_off1, sg_off, gm_off);
          entry(v1, idx_1, ok_1);
          load_tile<D, KK, VK>(B, kt, vt, kb, vb, k_off, klo_off, n_off, v_off, v_off1, sg_off, gm_off);
        };
        first_tiles();
  #pragma unroll
        for (int i = 0; i < NBT; ++i) s_bt[tid + kThreads * i] = btv[i];

        // -------- part 0 of each virtual head: rotate its 8 q rows once (row g
        // of the rotated q is H (s_K * q_g), unnormalised) and build its q.K B
        // operands: the scaled rotated q split into an fp16 high part (lanes
        // j < 8) and the fp16 rounding of the remainder (lanes j >= 8).  The
        // rows are staged in the virtual head's own operand area (8 rows of D
        // floats: its size), which the operands overwrite once every lane has
        // read its values.
        if (part == 0) {
          float* const stage = reinterpret_cast<float*>(qv_all + vh * NQK * 64);
          {
            float x[PER];
            if (p.q_f32) {
  #pragma unroll
              for (int e = 0; e < PER; ++e) x[e] = __uint_as_float(qw[e]);
            } else {
  #pragma unroll
              for (int k = 0; k < PER / 2; ++k) {
                x[2 * k] = __uint_as_float(qw[k] << 16);
                x[2 * k + 1] = __uint_as_float(qw[k] & 0xFFFF0000u);
              }
            }
            const uint32_t sw = s_par[20 + ((l8 * PER) >> 5)] >> ((l8 * PER) & 31);
  #pragma unroll
            for (int e = 0; e < PER; ++e) {
              if ((sw >> e) & 1u) x[e] = -x[e];
              if (!q_live) x[e] = 0.f;
            }
  #pragma unroll
            for (int h = 1; h < PER; h <<= 1) {
  #pragma unroll
              for (int e = 0; e < PER; ++e)
                if ((e & h) == 0) {
                  const float a0 = x[e], b0v = x[e + h];
                  x[e] = a0 + b0v;
                  x[e + h] = a0 - b0v;
                }
            }
            // the 3 stages across the 8 lanes of the row go through LDS: the
            // row is written in channel order, then lane l8 takes channels
            // PER k + PH l8 + m (k < 8, m < PH) and runs those stages in its
            // registers
            constexpr int PH = PER / 8;
            float* qrow = stage + g8 * D;
  #pragma unroll
            for (int i = 0; i < PER / 4; ++i)
              *reinterpret_cast<float4*>(qrow + l8 * PER + 4 * i) = float4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
            // the lanes of a row exchange values through LDS: a wave-scope
            // fence orders the writes above before the reads below
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            float y[8 * PH];
  #pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int c = PER * k + PH * l8;
              if constexpr (PH == 2) {
                const float2 f = *reinterpret_cast<const float2*>(qrow + c);
                y[2 * k] = f.x;
                y[2 * k + 1] = f.y;
              } else {
                y[k] = qrow[c];
              }
            }
  #pragma unroll
            for (int h = PH; h < 8 * PH; h <<= 1) {
  #pragma unroll
              for (int e = 0; e < 8 * PH; ++e)
                if ((e & h) == 0) {
                  const float a0 = y[e], b0v = y[e + h];
                  y[e] = a0 + b0v;
                  y[e + h] = a0 - b0v;
                }
            }
            float amax = 0.f;
  #pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int c = PER * k + PH * l8;
              if constexpr (PH == 2) *reinterpret_cast<float2*>(qrow + c) = float2{y[2 * k], y[2 * k + 1]};
              else qrow[c] = y[k];
            }
  #pragma unroll
            for (int e = 0; e < 8 * PH; ++e) amax = fmaxf(amax, fabsf(y[e]));
            amax = fmaxf(amax, lane_xor<1>(amax, ln));
            amax = fmaxf(amax, lane_xor<2>(amax, ln));
            amax = fmaxf(amax, lane_xor<4>(amax, ln));
            int ex = 0;
            if (amax > 0.f) frexpf(amax, &ex);
            if (l8 == 0) s_qexp[8 * vh + g8] = 15 - ex;   // amax * 2^(15-ex) in [2^14, 2^15)
          }
        }
        if constexpr (C::QJ) {
          // QJL: the projected rows u_g = S_g q_g of every virtual head (q_g:
          // the rotated row scaled by 2^(15-ex), group g's channels in listed
          // order) on the matrix cores, in 16-output tiles spread over all the
          // workgroup's waves: A = S (fp16 high and low parts of the fp32 values,
          // one MFMA each), B = the rows (high part in columns 0-7, low part in
          // 8-15), so each output sums all four cross products in fp32.  The u
          // rows go to the area of virtual head 8 + vh (at most 8 of them).
          lds_barrier();   // the rotated rows of every virtual head are staged
          const int lp = fresh_lane();
          const int pa = lp >> 4, pc = lp & 15;
          const int grp = (16 * ot_w) / QM;
          half8_t ah[QKC], al[QKC];   // A: S_grp[i][32 kc + 8 pa .. + 7], i = output 16 ot_w + pc of the group
  #pragma unroll
          for (int kc = 0; kc < QKC; ++kc) {
            const float sv[8] = {spf[2 * kc].x, spf[2 * kc].y, spf[2 * kc].z, spf[2 * kc].w,
                                 spf[2 * kc + 1].x, spf[2 * kc + 1].y, spf[2 * kc + 1].z, spf[2 * kc + 1].w};
  #pragma unroll
            for (int e = 0; e < 8; ++e) {
              ah[kc][e] = (_Float16)sv[e];
              al[kc][e] = (_Float16)(sv[e] - (float)ah[kc][e]);
            }
          }
          for (int vq = wave / QOT; vq < VH; vq += kWaves / QOT) {
            const float* rows = reinterpret_cast<const float*>(qv_all + vq * NQK * 64);
            float* const urows = reinterpret_cast<float*>(qv_all + (8 + vq) * NQK * 64);
            const float rpow = ldexpf(1.0f, s_qexp[8 * vq + (pc & 7)]);   // the column's row scale
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
            // listed channels of positions grp M + 32 kc + 8 pa .. + 7 (two-group
            // K: 8 bytes of the channel list, read at once for every kc)
            uint2 chw[QKC];
            if constexpr (C::MIXED) {
  #pragma unroll
              for (int kc = 0; kc < QKC; ++kc)
                chw[kc] = *reinterpret_cast<const uint2*>(s_par + 32 + ((grp * QM + 32 * kc + 8 * pa) >> 2));
            }
  #pragma unroll
            for (int kc = 0; kc < QKC; ++kc) {
              // B: values j = 32 kc + 8 pa + e of row pc & 7 (group order)
              half8_t bq;
  #pragma unroll
              for (int e = 0; e < 8; ++e) {
                int chn = grp * QM + 32 * kc + 8 * pa + e;
                if constexpr (C::MIXED) chn = (int)((((e >> 2) ? chw[kc].y : chw[kc].x) >> (8 * (e & 3))) & 0xFFu);
                const float v = rows[(pc & 7) * D + chn] * rpow;
                const _Float16 hi = (_Float16)v;
                bq[e] = (pc & 8) ? (_Float16)(v - (float)hi) : hi;
              }
              acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[kc], bq, acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[kc], bq, acc, 0, 0, 0);
            }
            // output 16 ot_w + 4 pa + e of row pc (columns pc and pc + 8 summed)
  #pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float u = acc[e] + row_ror8(acc[e]);
              if (pc < 8) urows[pc * D + 16 * ot_w + 4 * pa + e] = u;
            }
          }
          __syncthreads();   // every u row is written
        }
        if (part == 0) {
          float* const stage = reinterpret_cast<float*>(qv_all + vh * NQK * 64);
          // (lane roles recomputed from the fresh lane index: values kept
          // across the block loop may sit in scratch, whose reloads here would
          // wait for the tile loads in flight)
          const int la = ln >> 4, lq = ln & 7;
          const bool lo_q = (ln & 8) != 0;
          const float q_pow = ldexpf(1.0f, s_qexp[8 * vh + lq]);
          const float* qrow = stage + lq * D;
          // operand t of this lane: the 8 values it multiplies, scaled by
          // 2^(15-ex) and split into the fp16 high part (lanes j < 8) or the
          // fp16 rounding of the remainder (lanes j >= 8); all operands are
          // built in registers before any is written over the rows
          half8_t qvr[NQK];
          // two-group K: operand element (t, e) of lane (a, j) is channel
          // k_ch[pos] of the column, pos = (t / per_g) m + a (m / 4) + 8 (t %
          // per_g) + e; the 8 list bytes of each t are read at once, before
          // any row value
          uint2 chl[NQK];
          if constexpr (C::MIXED) {
            constexpr int m = D / 2;
            constexpr int per_g = NQK / 2;
  #pragma unroll
            for (int t = 0; t < NQK; ++t)
              chl[t] = *reinterpret_cast<const uint2*>(s_par + 32 + (((t / per_g) * m + la * (m / 4) + 8 * (t % per_g)) >> 2));
          }
  #pragma unroll
          for (int t = 0; t < NQK; ++t) {
            float vq[8];
            if constexpr (C::MIXED) {
  #pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int chn = (int)((((e >> 2) ? chl[t].y : chl[t].x) >> (8 * (e & 3))) & 0xFFu);
                vq[e] = qrow[chn];
              }
            } else {
  #pragma unroll
              for (int h = 0; h < 2; ++h) {
                const float4 f = *reinterpret_cast<const float4*>(qrow + la * (D / 4) + 8 * t + 4 * h);
                vq[4 * h] = f.x; vq[4 * h + 1] = f.y; vq[4 * h + 2] = f.z; vq[4 * h + 3] = f.w;
              }
            }
  #pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = vq[e] * q_pow;
              const _Float16 hi = (_Float16)v;
              const _Float16 lo = (_Float16)(v - (float)hi);
              qvr[t][e] = lo_q ? lo : hi;
            }
          }
          // every row read above is done before the operand writes below reuse
          // the bytes
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  #pragma unroll
          for (int t = 0; t < NQK; ++t) qv_all[(vh * NQK + t) * 64 + ln] = qvr[t];
          if constexpr (C::QJ) {
            // sketch operands: lane (a, j) multiplies outputs (D / 4) a + 8 t + e
            // of its column's u row (sign byte NQK a + t of a K row), scaled
            // by 2^(15-eu) (largest |u| of the row in [2^14, 2^15)) and split
            // into high and low fp16 parts like q
            const float* urow = reinterpret_cast<const float*>(qv_all + (8 + vh) * NQK * 64) + lq * D;
            float uv[NQK][8];
            float amax = 0.f;
  #pragma unroll
            for (int t = 0; t < NQK; ++t)
  #pragma unroll
              for (int h = 0; h < 2; ++h) {
                const float4 f = *reinterpret_cast<const float4*>(urow + la * (D / 4) + 8 * t + 4 * h);
                uv[t][4 * h] = f.x; uv[t][4 * h + 1] = f.y; uv[t][4 * h + 2] = f.z; uv[t][4 * h + 3] = f.w;
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
              }
            amax = fmaxf(amax, lane_xor<16>(amax, ln));
            amax = fmaxf(amax, lane_xor<32>(amax, ln));
            int eu = 0;
            if (amax > 0.f) frexpf(amax, &eu);
            const float u_pow = ldexpf(1.0f, 15 - eu);
            // the sketch's weight relative to the q.K sum: sqrt(pi / 2) / m
            // against 1 / sqrt(m) (both over sqrt(d)), and the two scalings
            if (ln < 8) s_rq[8 * vh + ln] = ldexpf(sqrtf(1.5707963267948966f / (float)(D / C::NGK)), eu - 15);
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // the u rows are read
  #pragma unroll
            for (int t = 0; t < NQK; ++t) {
              half8_t sv;
  #pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float v = uv[t][e] * u_pow;
                const _Float16 hi = (_Float16)v;
                sv[e] = lo_q ? (_Float16)(v - (float)hi) : hi;
              }
              qv_all[((8 + vh) * NQK + t) * 64 + ln] = sv;
            }
          }
        }
        lds_barrier();  // operands, counters and block-table entries ready
        TQ_MARK(3 + 4 * n_done);
        int ph2v = bt_at(idx_2);
        int g3 = grab();
        const float w_col = ldexpf(p.score_mul, -s_qexp[8 * vh + gq]);
        const half8_t* qb = qv_all + vh * NQK * 64 + lane;   // qb[64 * t]: operand of MFMA t
        const half8_t* qs = qv_all + (8 + vh) * NQK * 64 + lane;   // QJL: sketch operand t at qs[64 * t]
        const float r_col = C::QJ ? s_rq[8 * vh + gq] : 0.f;

        // -------- stream this wave's blocks of the piece
        // online softmax state per column: running max m_run (raw score
        // units), sum l_run and accumulator o_acc of the weights
        // 2^(w_col (s - m_run) + e_run); e_run (the same in every lane) is the
        // power of two that keeps p * n_V * 2^e_run in fp16's normal range:
        // 15 - ex, 2^(ex-1) <= the largest V norm so far < 2^ex (39 before any)
        float m_run = -INFINITY, l_run = 0.f;
        int e_run = 39;
        uint32_t v_hi = v_bound_m1(39);
        float nm = 39.f;   // exp2 offset: e_run - w_col m_run (e_run while m_run is -inf)
        float4_t o_acc[C::R];
  #pragma unroll
        for (int u = 0; u < C::R; ++u) o_acc[u] = float4_t{0.f, 0.f, 0.f, 0.f};

        // token r's V bytes of this lane, from byte 0 (r compile-time)
        auto vword = [&](const Tile<D, KK, VK>& t, int r) -> uint32_t {
          if constexpr (C::VLANE == 4) return t.v[r];
          else if constexpr (C::VLANE == 2) return (r & 1) ? (t.v[r >> 1] >> 16) : t.v[r >> 1];
          else return t.v[0] >> (8 * r);
        };
        auto compute = [&](const Tile<D, KK, VK>& cur, int b, bool ok) {
          float4_t acc0 = {0.f, 0.f, 0.f, 0.f};
          float4_t acc1 = {0.f, 0.f, 0.f, 0.f};
          if constexpr (C::KB == K4) {
  #pragma unroll
            for (int t = 0; t < NQK; ++t) {
              u32x4_t av;
  #pragma unroll
              for (int by = 0; by < 4; ++by) av[by] = lds_u32(lds, lut_addr(cur.k[t], off4_k, by));
              acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qb[64 * t], acc0, 0, 0, 0);
            }
          } else if constexpr (C::KB == K2) {
  #pragma unroll
            for (int t = 0; t < NQK; ++t) {
              const uint2 x0 = lds_u64(lds, lut_addr(cur.k[t >> 1], off2_k, 2 * (t & 1)));
              const uint2 x1 = lds_u64(lds, lut_addr(cur.k[t >> 1], off2_k, 2 * (t & 1) + 1));
              const u32x4_t av = {x0.x, x0.y, x1.x, x1.y};
              acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qb[64 * t], acc0, 0, 0, 0);
            }
          } else if constexpr (C::KB == KM43) {   // 4-bit group 0 by the nibble table, 3-bit group 1 by the pair table
            constexpr int per_g = NQK / 2;
  #pragma unroll
            for (int u = 0; u < per_g; ++u) {
              u32x4_t av;
  #pragma unroll
              for (int by = 0; by < 4; ++by) av[by] = lds_u32(lds, lut_addr(cur.k[u], off4_k, by));
              acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qb[64 * u], acc0, 0, 0, 0);
            }
            constexpr int LB = 3 * D / 64;
            const int lo_off = tokK * C::KROW + D / 4 + LB * a;
            const uint64_t win = ((uint64_t)cur.k_lo[1] << 32 | cur.k_lo[0]) >> ((lo_off & 3) * 8);
  #pragma unroll
            for (int u = 0; u < per_g; ++u) {
              u32x4_t av;
  #pragma unroll
              for (int pr = 0; pr < 4; ++pr) {
                const uint32_t key = (uint32_t)(win >> (6 * (4 * u + pr))) & 63u;
                av[pr] = lds_u32(lds, (key << 6) | off3);
              }
              acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qb[64 * (per_g + u)], acc1, 0, 0, 0);
            }
          } else {   // 3 + 2 bits: 3-bit group 0 by the pair table, 2-bit group 1 by the crumb table
            constexpr int per_g = NQK / 2;
            constexpr int LB = 3 * D / 64;
            const int g0_off = tokK * C::KROW + LB * a;
            const uint64_t win = ((uint64_t)cur.k_lo[1] << 32 | cur.k_lo[0]) >> ((g0_off & 3) * 8);
  #pragma unroll
            for (int u = 0; u < per_g; ++u) {
              u32x4_t av;
  #pragma unroll
              for (int pr = 0; pr < 4; ++pr) {
                const uint32_t key = (uint32_t)(win >> (6 * (4 * u + pr))) & 63u;
                av[pr] = lds_u32(lds, (key << 6) | off3);
              }
              acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qb[64 * u], acc0, 0, 0, 0);
            }
            const int g1_off = tokK * C::KROW + 3 * D / 16 + (D / 32) * a;
            const uint32_t kw = cur.k[0] >> ((g1_off & 3) * 8);
  #pragma unroll
            for (int u = 0; u < per_g; ++u) {
              const uint2 x0 = lds_u64(lds, lut_addr(kw, off2_k, 2 * u));
              const uint2 x1 = lds_u64(lds, lut_addr(kw, off2_k, 2 * u + 1));
              const u32x4_t av = {x0.x, x0.y, x1.x, x1.y};
              acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qb[64 * (per_g + u)], acc1, 0, 0, 0);
            }
          }

          // stage boundary: keeps the scheduler from hoisting the next stage's
          // table reads above these MFMAs (bounds the live registers)
          __builtin_amdgcn_sched_barrier(0);
          const int tok0 = 16 * b;
          const bool part = !(ok && tok0 + 16 <= ctx_all);   // partial or skipped block (wave-uniform)
          // tokens a + 4e of this lane that count (all, unless part)
          auto live = [&](int e) { return ok && (tok0 + a + 4 * e) < ctx_col; };
          // raw scores of this lane's 4 tokens for q head gq: sr = (q . c) * n_K;
          // the exp2-domain score is w_col * sr (w_col > 0), folded into one fma
          float sc[4];
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float full0 = acc0[e] + row_ror8(acc0[e]);
            const uint32_t kw = (e >> 1) ? cur.kn[0].y : cur.kn[0].x;
            float v = (e & 1) ? mul_h<1>(full0, kw) : mul_h<0>(full0, kw);
            if constexpr (C::MIXED) {
              const float full1 = acc1[e] + row_ror8(acc1[e]);
              const uint32_t kw1 = (e >> 1) ? cur.kn[1].y : cur.kn[1].x;
              v = (e & 1) ? fma_h<1>(full1, kw1, v) : fma_h<0>(full1, kw1, v);
            }
            sc[e] = v;
          }
          if constexpr (C::QJ) {
            // QJL: the sketch sum of this lane's K row against the projected
            // query (after the q.K sums are consumed, so that its accumulator
            // reuses their registers), one MFMA per 32 outputs with A =
            // +-(residual norm) in fp16 (exact): sign bit e2 of a byte to bit
            // 15, bit e2 + 1 to bit 31 of the operand dword
            float4_t accq = {0.f, 0.f, 0.f, 0.f};
            const int lq = fresh_lane();
            const uint32_t sb_all = cur.sg >> (8 * ((NQK * (lq >> 4)) & 3));
            const uint32_t gam = (cur.gm >> (16 * (lq & 1))) & 0xFFFFu;
            const uint32_t g2 = gam | (gam << 16);
  #pragma unroll
            for (int t = 0; t < NQK; ++t) {
              const uint32_t sb = (sb_all >> (8 * t)) & 0xFFu;
              const uint32_t spread = sb | (sb << 15);
              u32x4_t av;
  #pragma unroll
              for (int e2 = 0; e2 < 4; ++e2) av[e2] = ((spread << (15 - 2 * e2)) & 0x80008000u) | g2;
              accq = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qs[64 * t], accq, 0, 0, 0);
            }
  #pragma unroll
            for (int e = 0; e < 4; ++e) sc[e] = __builtin_fmaf(accq[e] + row_ror8(accq[e]), r_col, sc[e]);
          }
          if (part) {
  #pragma unroll
            for (int e = 0; e < 4; ++e) sc[e] = live(e) ? sc[e] : -INFINITY;
          }
          const float bm = max_rows(max_nn(max_nn(sc[0], sc[1]), max_nn(sc[2], sc[3])));
          const float m_new = max_nn(m_run, bm);
          // a V norm of this lane's tokens too large for the current e_run?
          // (masked tokens' norm bytes may hold anything: left out)
          u16x2_t mxv = __builtin_elementwise_max(as_u16x2(cur.vn[0].x), as_u16x2(cur.vn[0].y));
          if constexpr (C::MIXED_V)
            mxv = __builtin_elementwise_max(mxv, __builtin_elementwise_max(as_u16x2(cur.vn[1].x), as_u16x2(cur.vn[1].y)));
          if (part) {
            mxv = u16x2_t{0, 0};
  #pragma unroll
            for (int g = 0; g < C::NVG; ++g) {
              uint32_t vx = cur.vn[g].x, vy = cur.vn[g].y;
  #pragma unroll
              for (int e = 0; e < 4; ++e)
                if (!live(e)) {
                  if (e >> 1) vy &= ~(0xFFFFu << (16 * (e & 1)));
                  else vx &= ~(0xFFFFu << (16 * (e & 1)));
                }
              mxv = __builtin_elementwise_max(mxv, __builtin_elementwise_max(as_u16x2(vx), as_u16x2(vy)));
            }
          }
          const bool over = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(mxv, u16x2_t{(uint16_t)v_hi, (uint16_t)v_hi})) != 0u;
          if (__builtin_amdgcn_ballot_w64((m_new > m_run) | over)) {
            asm volatile("" ::: "memory");   // keep this a real (rarely taken) branch
            int e_new = e_run;
            if (__builtin_amdgcn_ballot_w64(over)) {
              // 15 - ex for the largest V norm of the tile (all 16 tokens),
              // capped at the largest finite fp16
              const uint32_t mh = mxv[0] > mxv[1] ? mxv[0] : mxv[1];
              const float nmax = fminf(max_rows(f16_exact<0>(mh)), 65504.f);
              const int ex = uni((int)((__float_as_uint(nmax) >> 23) & 0xFF) - 126);
              e_new = 15 - ex < e_run ? 15 - ex : e_run;
              v_hi = v_bound_m1(e_new);
            }
            const float sh = (float)(e_new - e_run);   // <= 0
            const float alpha = __builtin_amdgcn_exp2f((m_new > m_run) ? __builtin_fmaf(m_run - m_new, w_col, sh) : sh);
            l_run *= alpha;
  #pragma unroll
            for (int u = 0; u < C::R; ++u) o_acc[u] *= alpha;
            m_run = m_new;
            e_run = e_new;
            nm = (m_run == -INFINITY) ? (float)e_run : __builtin_fmaf(-m_run, w_col, (float)e_run);
          }
          float pr[4];
  #pragma unroll
          for (int e = 0; e < 4; ++e) pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], w_col, nm));   // -inf -> 0
          l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);

          // P.V on the matrix cores: A = V (dims x tokens) per MFMA i, through
          // `into(i, A)` (i compile-time)
          auto pv = [&](auto&& into) {
            if constexpr (C::MIXED_V) {
              // two groups: MFMAs 0 .. PPL-1 take group 0, PPL .. 2 PPL-1 group
              // 1; MFMA (g, i) row r is position 8 (r % OCT) + (r / OCT) PPL + i
              // of group g, so this lane's codes of token e sit at index
              // (lane & 15) / OCT * PPL + i of the token's octet in its run
              const int sub = (fresh_lane() & 15) / C::OCT;
              auto group = [&](auto bk, const uint32_t* w, auto base) {
                constexpr int b = decltype(bk)::value;
                constexpr int I0 = decltype(base)::value;
                if constexpr (b == 4) {
                  // octet of token e = word e (8 nibbles); nibbles sub PPL + i,
                  // paired across tokens as in the one-group 4-bit path
                  const uint32_t sh = (uint32_t)(4 * C::PPL * sub);
                  const uint32_t w0 = w[0] >> sh, w1 = w[1] >> sh, w2 = w[2] >> sh, w3 = w[3] >> sh;
                  const uint32_t E01 = (w0 & 0x0F0F0F0Fu) | ((w1 << 4) & 0xF0F0F0F0u);
                  const uint32_t O01 = ((w0 >> 4) & 0x0F0F0F0Fu) | (w1 & 0xF0F0F0F0u);
                  const uint32_t E23 = (w2 & 0x0F0F0F0Fu) | ((w3 << 4) & 0xF0F0F0F0u);
                  const uint32_t O23 = ((w2 >> 4) & 0x0F0F0F0Fu) | (w3 & 0xF0F0F0F0u);
  #pragma unroll
                  for (int i = 0; i < C::PPL; ++i) {
                    const u32x2_t av = {lds_u32(lds, lut_addr((i & 1) ? O01 : E01, off_v4, i >> 1)),
                                        lds_u32(lds, lut_addr((i & 1) ? O23 : E23, off_v4, i >> 1))};
                    into(I0 + i, __builtin_bit_cast(half4_t, av));
                  }
                } else if constexpr (b == 3) {
                  // octet of token e = bits 24 e .. 24 e + 23 of the 3 words;
                  // keys of the pair table: code(t0) | code(t1) << 3
                  const uint32_t sh = (uint32_t)(3 * C::PPL * sub);
                  const uint32_t x0 = w[0] >> sh;
                  const uint32_t x1 = __builtin_amdgcn_alignbit(w[1], w[0], 24) >> sh;
                  const uint32_t x2 = __builtin_amdgcn_alignbit(w[2], w[1], 16) >> sh;
                  const uint32_t x3 = (w[2] >> 8) >> sh;
  #pragma unroll
                  for (int i = 0; i < C::PPL; ++i) {
                    const uint32_t k01 = ((x0 >> (3 * i)) & 7u) | (((x1 >> (3 * i)) & 7u) << 3);
                    const uint32_t k23 = ((x2 >> (3 * i)) & 7u) | (((x3 >> (3 * i)) & 7u) << 3);
                    const u32x2_t av = {lds_u32(lds, (k01 << 6) | off3), lds_u32(lds, (k23 << 6) | off3)};
                    into(I0 + i, __builtin_bit_cast(half4_t, av));
                  }
                } else {
                  // octet of token e = half-word e of the 2 words (8 crumbs);
                  // crumbs sub PPL + i of the 4 tokens transposed so that byte i
                  // holds position i of tokens 0-3: the crumb table returns the
                  // operand's 4 values in token order
                  const uint32_t sh = (uint32_t)(2 * C::PPL * sub);
                  const uint32_t y = ((w[0] >> sh) & 0xFFu) | (((w[0] >> 16 >> sh) & 0xFFu) << 8) |
                                     (((w[1] >> sh) & 0xFFu) << 16) | (((w[1] >> 16 >> sh) & 0xFFu) << 24);
                  uint32_t t = (y ^ (y >> 6)) & 0x00CC00CCu;
                  uint32_t x = y ^ t ^ (t << 6);
                  t = (x ^ (x >> 12)) & 0x0000F0F0u;
                  x = x ^ t ^ (t << 12);
  #pragma unroll
                  for (int i = 0; i < C::PPL; ++i) {
                    const uint2 l4 = lds_u64(lds, lut_addr(x, off_v2, i));
                    into(I0 + i, __builtin_bit_cast(half4_t, u32x2_t{l4.x, l4.y}));
                  }
                }
              };
              group(std::integral_constant<int, C::VB0>{}, cur.v, std::integral_constant<int, 0>{});
              group(std::integral_constant<int, C::VB1>{}, cur.v + C::VB0, std::integral_constant<int, C::PPL>{});
            } else if constexpr (VK == V4) {
              // Lookup keys pair the nibbles of two tokens for one dim, so the
              // nibble table returns the MFMA operand dword (V[t0][d], V[t1][d])
              // directly: byte k of E holds dim 2k, byte k of Od dim 2k+1.
              const uint32_t w0 = vword(cur, 0), w1 = vword(cur, 1), w2 = vword(cur, 2), w3 = vword(cur, 3);
              const uint32_t x1s = w1 << 4, x3s = w3 << 4;
              const uint32_t E01 = (w0 & 0x0F0F0F0Fu) | (x1s & 0xF0F0F0F0u);
              const uint32_t O01 = ((w0 >> 4) & 0x0F0F0F0Fu) | (w1 & 0xF0F0F0F0u);
              const uint32_t E23 = (w2 & 0x0F0F0F0Fu) | (x3s & 0xF0F0F0F0u);
              const uint32_t O23 = ((w2 >> 4) & 0x0F0F0F0Fu) | (w3 & 0xF0F0F0F0u);
              constexpr int NB = D / 32;  // bytes per token in this lane (2 dims each)
  #pragma unroll
              for (int k = 0; k < NB; ++k) {
  #pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                  const u32x2_t av = {lds_u32(lds, lut_addr(hh ? O01 : E01, off_v4, k)),
                                      lds_u32(lds, lut_addr(hh ? O23 : E23, off_v4, k))};
                  into(2 * k + hh, __builtin_bit_cast(half4_t, av));
                }
              }
            } else {
              constexpr int NBY = D / 64;  // bytes per token in this lane (4 dims each)
  #pragma unroll
              for (int k = 0; k < NBY; ++k) {
                uint2 lk[4];
  #pragma unroll
                for (int r = 0; r < 4; ++r) {
                  // byte k of token r: word r / 2, byte 2 (r % 2) + k (2-byte runs) or byte r (1-byte runs)
                  if constexpr (C::VLANE == 2) lk[r] = lds_u64(lds, lut_addr(cur.v[r >> 1], off_v2, 2 * (r & 1) + k));
                  else lk[r] = lds_u64(lds, lut_addr(cur.v[0], off_v2, r + k));
                }
  #pragma unroll
                for (int t = 0; t < 4; ++t) {
                  const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
                  const uint32_t w0 = (t >> 1) ? lk[0].y : lk[0].x;
                  const uint32_t w1 = (t >> 1) ? lk[1].y : lk[1].x;
                  const uint32_t w2 = (t >> 1) ? lk[2].y : lk[2].x;
                  const uint32_t w3 = (t >> 1) ? lk[3].y : lk[3].x;
                  const u32x2_t av = {__builtin_amdgcn_perm(w1, w0, sel), __builtin_amdgcn_perm(w3, w2, sel)};
                  into(4 * k + t, __builtin_bit_cast(half4_t, av));
                }
              }
            }
          };
          // B operand: p * n_V in fp16 (p carrying 2^e_run), each rounded once
          // (two V groups: one operand per group's norms)
          half4_t pb[C::NVG];
  #pragma unroll
          for (int g = 0; g < C::NVG; ++g) {
            u32x2_t pw = {mul_h2(pr[0], pr[1], cur.vn[g].x), mul_h2(pr[2], pr[3], cur.vn[g].y)};
            if (part) {
              // a masked token's weight is 0, but its norm bytes may hold any
              // bits (a NaN times 0 is NaN): its operand is set to +0
  #pragma unroll
              for (int e = 0; e < 4; ++e)
                if (!live(e)) pw[e >> 1] &= ~(0xFFFFu << (16 * (e & 1)));
            }
            pb[g] = __builtin_bit_cast(half4_t, pw);
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (C::KB == KM32) {
            // every V operand of the tile is looked up before the first P.V
            // MFMA (one LDS round trip per tile instead of one per MFMA);
            // measured faster with the 3+2-bit K recipe only (with the other
            // K kinds the same order is no faster or slower)
            half4_t va[C::R];
            pv([&](int i, half4_t av) { va[i] = av; });
            __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
            for (int i = 0; i < C::R; ++i)
              o_acc[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(va[i], pb[C::MIXED_V && i >= C::PPL ? 1 : 0], o_acc[i], 0, 0, 0);
          } else {
            pv([&](int i, half4_t av) {
              o_acc[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, pb[C::MIXED_V && i >= C::PPL ? 1 : 0], o_acc[i], 0, 0, 0);
            });
          }
        };

        // one block (j): issue tile j+2, look up the entry of j+3 and take the
        // index of j+4, compute tile j
        auto step = [&](const Tile<D, KK, VK>& cur, Tile<D, KK, VK>& dst) -> bool {
          if (idx_c >= n) return false;
          bool ok2;
          entry(ph2v, idx_2, ok2);
          load_tile<D, KK, VK>(dst, kt, vt, kb, vb, k_off, klo_off, n_off, v_off, v_off1, sg_off, gm_off);
          const int idx_3 = __builtin_amdgcn_readfirstlane(g3);
          const int ph3v = bt_at(idx_3);
          g3 = grab();
          compute(cur, b0 + idx_c, ok_c);
          idx_c = idx_1; ok_c = ok_1;
          idx_1 = idx_2; ok_1 = ok2;
          idx_2 = idx_3; ph2v = ph3v;
          return true;
        };
        for (;;) {
          if (!step(A, C3)) break;
          if (!step(B, A)) break;
          if (!step(C3, B)) break;
        }

        // -------- wave states to LDS (rotated domain): wave w stores its
        // unnormalised O rows (q head g at slot row 8 w + g) and its running
        // max / sum per q head
        __syncthreads();  // every wave is done with the q operands (the slots overlay them)
        TQ_MARK(4 + 4 * n_done);
        const int le = fresh_lane();
        l_run += lane_xor<16>(l_run, le);
        l_run += lane_xor<32>(l_run, le);
        if (!lo_part) {
          if constexpr (C::MIXED_V) {
            // accumulator (i, e) is position 8 (rho % OCT) + (rho / OCT) PPL +
            // i % PPL of V group i / PPL, rho = 4 a + e: stored at its channel
            float* srow = slots + (8 * wave + gq) * C::DS;
  #pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int rho = 4 * a + e;
  #pragma unroll
              for (int i = 0; i < C::R; ++i) {
                const int pos = (i / C::PPL) * (D / 2) + 8 * (rho % C::OCT) + (rho / C::OCT) * C::PPL + i % C::PPL;
                const int ch = (int)((s_vch[pos >> 2] >> (8 * (pos & 3))) & 0xFFu);
                srow[ch] = o_acc[i][e];
              }
            }
          } else {
            float* srow = slots + (8 * wave + gq) * C::DS + R4 * a;
  #pragma unroll
            for (int e = 0; e < 4; ++e)
  #pragma unroll
              for (int h = 0; h < C::R / 4; ++h)
                *reinterpret_cast<float4*>(srow + C::R * e + 4 * h) =
                    float4{o_acc[4 * h][e], o_acc[4 * h + 1][e], o_acc[4 * h + 2][e], o_acc[4 * h + 3][e]};
          }
          if (a == 0) {   // the exp2-domain offset of the weights (-inf: no token), and their sum
            s_ml[16 * wave + gq] = m_run == -INFINITY ? -INFINITY : -nm;
            s_ml[16 * wave + 8 + gq] = l_run;
          }
        }
        __syncthreads();

        // -------- combine the parts of each (virtual head, column) pair,
        // normalise, inverse rotation, write.  The pairs (CV columns per
        // virtual head) are taken 64 at a time; wave w takes pairs 4 w .. 4 w +
        // 3 of each round, 16 lanes each.  Lane m of a pair first holds dims m
        // + 16 k (k < D / 16) and runs the transform stages over k in its
        // registers, passes the row through LDS, then holds dims (D / 16) m + k,
        // runs the stages over k again and the remaining ones across the lanes
        // of the pair.
        const int CV = CG == 1 ? p.G : 8;
        const int npair = VH * CV;
        for (int pbase = 4 * wave; pbase < npair; pbase += 4 * kWaves) {
          constexpr int ND = D / 16;
          const int m = le & 15;
          const int pr_raw = pbase + (le >> 4);
          const int pr = pr_raw < npair ? pr_raw : npair - 1;
          const int h2 = CG == 1 ? (int)(((float)pr + 0.5f) * p.inv_G) : pr >> 3;   // virtual head: pr / CV (pr < 128)
          const int g = pr - h2 * CV;
          const int hk = h2 / CG;                   // its kv head of the group
          const int col = 8 * (h2 - hk * CG) + g;   // its column of the kv head
          const bool live = pr_raw < npair && col < p.G;
          float M = -INFINITY;   // wave states: weights 2^(w s - X_w), sums l_w
          for (int q = 0; q < NPW; ++q) M = fmaxf(M, s_ml[16 * wave_of_part(h2, q, VH) + g]);
          float y[ND];
  #pragma unroll
          for (int k = 0; k < ND; ++k) y[k] = 0.f;
          float L = 0.f;
          for (int q = 0; q < NPW; ++q) {
            const int wq = wave_of_part(h2, q, VH);
            const float mw = s_ml[16 * wq + g];
            const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            L = __builtin_fmaf(f, s_ml[16 * wq + 8 + g], L);
            const float* srow = slots + (8 * wq + g) * C::DS + m;
  #pragma unroll
            for (int k = 0; k < ND; ++k) y[k] = __builtin_fmaf(f, srow[16 * k], y[k]);
          }
  #pragma unroll
          for (int h = 1; h < ND; h <<= 1) {
  #pragma unroll
            for (int e = 0; e < ND; ++e)
              if ((e & h) == 0) {
                const float a0 = y[e], b0v = y[e + h];
                y[e] = a0 + b0v;
                y[e + h] = a0 - b0v;
              }
          }
          // the row of part 0 is read only by this pair's lanes, each lane
          // rewrites the dims it read; the fence below orders those writes
          // before the reads of the other lanes' dims
          float* row = slots + (8 * wave_of_part(h2, 0, VH) + g) * C::DS;
  #pragma unroll
          for (int k = 0; k < ND; ++k) row[m + 16 * k] = y[k];
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // other lanes' values below
  #pragma unroll
          for (int k = 0; k < ND; k += 4) {
            const float4 f = *reinterpret_cast<const float4*>(row + ND * m + k);
            y[k] = f.x; y[k + 1] = f.y; y[k + 2] = f.z; y[k + 3] = f.w;
          }
  #pragma unroll
          for (int h = 1; h < ND; h <<= 1) {
  #pragma unroll
            for (int e = 0; e < ND; ++e)
              if ((e & h) == 0) {
                const float a0 = y[e], b0v = y[e + h];
                y[e] = a0 + b0v;
                y[e + h] = a0 - b0v;
              }
          }
          wht_lanes<1>(y, le);   // dim bit 3 (D = 128) or bits 2, 3 (D = 64)
          if constexpr (ND == 4) wht_lanes<2>(y, le);
          const bool empty = !(L > 0.f);
          const float inv_sqrt_d = D == 128 ? 0.08838834764831845f : 0.125f;
          const float scale = empty ? 0.f : inv_sqrt_d * p.v_mul / L;
          const float lse = empty ? -INFINITY : (M + log2f(L)) * kLn2;
          const int qi = (int)(((float)col + 0.5f) * p.inv_Gr);   // column col = (query qi, q head col - qi Gr)
          const int64_t rowq = ((int64_t)s * p.NQ + qi) * p.Hq + (grp * HG + hk) * p.Gr + (col - qi * p.Gr);
          const int d0 = ND * m;
          const uint32_t sgn = s_par[24 + (d0 >> 5)] >> (d0 & 31);
  #pragma unroll
          for (int k = 0; k < ND; ++k) {
            const float sv = y[k] * scale;
            y[k] = ((sgn >> k) & 1u) ? -sv : sv;
          }
          if (live) {
            if (whole) {
              const int64_t off = rowq * D + d0;
              if (p.out_f32) {
  #pragma unroll
                for (int k = 0; k < ND; k += 4)
                  *reinterpret_cast<float4*>(static_cast<float*>(p.out) + off + k) = float4{y[k], y[k + 1], y[k + 2], y[k + 3]};
              } else {
                uint32_t w[ND / 2];
  #pragma unroll
                for (int k = 0; k < ND / 2; ++k)
                  w[k] = (uint32_t)f32_to_bf16_rne(y[2 * k]) | ((uint32_t)f32_to_bf16_rne(y[2 * k + 1]) << 16);
                uint16_t* o16 = static_cast<uint16_t*>(p.out) + off;
                if constexpr (ND == 8) *reinterpret_cast<uint4*>(o16) = uint4{w[0], w[1], w[2], w[3]};
                else *reinterpret_cast<uint2*>(o16) = uint2{w[0], w[1]};
              }
              if (m == 0 && p.lse) p.lse[rowq] = lse;
              if (m == 0 && p.P > 1) p.part_lse[rowq * p.PS] = __uint_as_float(kDoneBits);
            } else {
              const int64_t row0 = rowq * p.PS;
              const int64_t prow = row0 + piece;
  #pragma unroll
              for (int k = 0; k < ND; k += 4)
                *reinterpret_cast<float4*>(p.part_o + prow * D + d0 + k) = float4{y[k], y[k + 1], y[k + 2], y[k + 3]};
              if (m == 0) p.part_lse[prow] = lse;
              if (piece == n_pieces - 1)   // the last piece closes the slots no piece uses
                for (int i = n_pieces + m; i < p.P; i += 16) p.part_lse[row0 + i] = -INFINITY;
            }
          }
        }
        TQ_MARK(5 + 4 * n_done);
        ++n_done;
      }

      // -------- next segment
      pos = vb0 + nb_s;
      if (pos >= r1) break;
      off = 0;
      if (++grp == p.NG) {
        grp = 0;
        do {
          ++s;
          nb_s = (seq_len(p, s_cl, s) + 15) >> 4;
        } while (nb_s == 0);
      }
    }
  }
  window_items();
  TQ_MARK(14);
  TQ_MARK_VALUE(15, (uint64_t)n_done);
  (void)n_done;
}

// ----------------------------------------------------------------- merge
// One workgroup per (sequence, q head) row: out = sum_i exp(lse_i - M) o_i /
// sum_i exp(lse_i - M), lse = M + log(sum_i exp(lse_i - M)), M = max lse_i,
// over the P partial slots; a -inf lse marks an empty or unused slot.  In
// decode mode the decode kernel has marked the rows it wrote out directly
// (kDoneBits in slot 0) and set the slots past a segment's last piece to
// -inf, so no segment bookkeeping is redone here.  Every wave reads the lse
// of slots 0-63 (lane l: slot l).  With one wave (P <= 16) it then reads the
// o rows of the live slots only.  With NW = ceil(P / 16) > 1 waves (up to 4)
// each wave reads the o rows of its own 16 slots (wave w: slots 16 w ..)
// together with the lse, before the slots are known to be live (dead slots
// hold stale values that get weight 0), so a row with up to 64 pieces costs
// one memory round trip; slots past 16 NW are read once their lse values
// are known.  The waves' weighted sums are added in LDS.
struct MergeParams {
  const float* part_o;
  const float* part_lse;
  void* out;
  float* lse;
  int32_t S, H, P, D, out_f32, decode;
};

template <int NW>
__global__ __launch_bounds__(64 * NW) void merge_kernel(MergeParams p) {
  // one wave (P <= 16): the o rows are read once the lse values are in, and
  // only for live slots (a cut segment's pieces; the rest hold -inf), which
  // halves the bytes read at the 8B shape for one more short round trip;
  // more waves: every wave's first 16 o rows are requested with the lse
  constexpr bool LIVE = NW == 1;
  constexpr int CH = 16;
  __shared__ float red[NW > 1 ? NW - 1 : 1][2 * 64 + 1];
  const int64_t sh = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int P = p.P, D = p.D;
  const float* lse_p = p.part_lse + sh * P;
  const float* o_p = p.part_o + sh * (int64_t)P * D;
  const float lf = lane < P ? lse_p[lane] : -INFINITY;
  float ov0[CH][2];
  if constexpr (!LIVE) {
#pragma unroll
    for (int k = 0; k < CH; ++k)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int dim = lane + 64 * r;
        const int slot = CH * w + k;
        ov0[k][r] = (slot < P && dim < D) ? o_p[(int64_t)slot * D + dim] : 0.f;
      }
  }
  if (p.decode && (uint32_t)__builtin_amdgcn_readfirstlane(__float_as_uint(lf)) == kDoneBits) return;
  if constexpr (LIVE) {
    const uint64_t live = __builtin_amdgcn_ballot_w64(lane < P && lf != -INFINITY);
#pragma unroll
    for (int k = 0; k < CH; ++k)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int dim = lane + 64 * r;
        ov0[k][r] = (((live >> k) & 1) && dim < D) ? o_p[(int64_t)k * D + dim] : 0.f;
      }
  }
  auto slot_lse = [&](int i) -> float {   // i uniform
    return i < 64 ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(lf), i)) : lse_p[i];
  };
  float M = lf;
  for (int i = 64 + lane; i < P; i += 64) M = fmaxf(M, lse_p[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float acc[2] = {0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {
    for (int base = CH * w; base < P; base += CH * NW) {
      float wt[CH], ov[CH][2];
#pragma unroll
      for (int k = 0; k < CH; ++k) {   // all loads of the chunk before any use
        const float li = base + k < P ? slot_lse(base + k) : -INFINITY;
        wt[k] = li;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int dim = lane + 64 * r;
          ov[k][r] = base == CH * w ? ov0[k][r]
                                    : ((li != -INFINITY && dim < D) ? o_p[(int64_t)(base + k) * D + dim] : 0.f);
        }
      }
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const float wk = (wt[k] == -INFINITY) ? 0.f : expf(wt[k] - M);
        den += wk;
#pragma unroll
        for (int r = 0; r < 2; ++r) acc[r] = wk > 0.f ? __builtin_fmaf(wk, ov[k][r], acc[r]) : acc[r];
      }
    }
  }
  if constexpr (NW > 1) {   // add the other waves' sums to wave 0's
    if (w > 0) {
      red[w - 1][lane] = acc[0];
      red[w - 1][64 + lane] = acc[1];
      if (lane == 0) red[w - 1][128] = den;
    }
    __syncthreads();
    if (w > 0) return;
#pragma unroll
    for (int v = 0; v < NW - 1; ++v) {
      acc[0] += red[v][lane];
      acc[1] += red[v][64 + lane];
      den += red[v][128];
    }
  }
  const bool empty = !(den > 0.f);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int dim = lane + 64 * r;
    if (dim >= D) continue;
    const float o = empty ? 0.f : acc[r] / den;
    const int64_t off = sh * D + dim;
    if (p.out_f32) static_cast<float*>(p.out)[off] = o;
    else static_cast<uint16_t*>(p.out)[off] = f32_to_bf16_rne(o);
  }
  if (lane == 0 && p.lse) p.lse[sh] = empty ? -INFINITY : M + logf(den);
}

// One workgroup per row, ceil(P / 16) waves (at most 4).
void launch_merge(const MergeParams& mp, int64_t rows, hipStream_t st) {
  const dim3 grid((unsigned)rows);
  if (mp.P > 48) hipLaunchKernelGGL(merge_kernel<4>, grid, dim3(256), 0, st, mp);
  else if (mp.P > 32) hipLaunchKernelGGL(merge_kernel<3>, grid, dim3(192), 0, st, mp);
  else if (mp.P > 16) hipLaunchKernelGGL(merge_kernel<2>, grid, dim3(128), 0, st, mp);
  else hipLaunchKernelGGL(merge_kernel<1>, grid, dim3(64), 0, st, mp);
}

template <int D, int KK, int VK>
void launch_decode(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<D, KK, VK>), dim3((unsigned)p.n_wg), dim3(kThreads), 0, st, p);
}

int format_kind_k(const tq_format* f) {
  if (f->num_groups == 1 && f->group_bits[0] == 4) return K4;
  if (f->num_groups == 1 && f->group_bits[0] == 2) return K2;
  if (f->num_groups == 2 && f->group_bits[0] == 4 && f->group_bits[1] == 3) return KM43;
  if (f->num_groups == 2 && f->group_bits[0] == 3 && f->group_bits[1] == 2) return KM32;
  return -1;
}

int format_kind_v(const tq_format* f) {
  if (f->num_groups == 1 && f->group_bits[0] == 4) return V4;
  if (f->num_groups == 1 && f->group_bits[0] == 2) return V2;
  if (f->num_groups == 2 && f->group_bits[0] == 4 && f->group_bits[1] == 3) return VM43;
  if (f->num_groups == 2 && f->group_bits[0] == 3 && f->group_bits[1] == 2) return VM32;
  return -1;
}

}  // namespace
}  // namespace tq

using namespace tq;

#ifdef TQ_PHASE_TRACE
static uint64_t* g_phase_trace = nullptr;
#endif

extern "C" tq_status tq_debug_phase_trace(uint64_t* buf) {
#ifdef TQ_PHASE_TRACE
  __atomic_store_n(&g_phase_trace, buf, __ATOMIC_RELEASE);
  return TQ_OK;
#else
  (void)buf;
  return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "library built without TQ_PHASE_TRACE");
#endif
}

extern "C" tq_status tq_split_merge(const float* part_out, const float* part_lse, int32_t num_seqs,
                                    int32_t num_heads, int32_t num_splits, int32_t head_dim, void* out,
                                    tq_dtype out_dtype, float* lse, tq_stream_t stream) {
  if (num_seqs < 0 || num_heads <= 0 || num_splits <= 0) return set_error(TQ_ERR_VALUE, "bad merge shape");
  if (head_dim != 64 && head_dim != 128) return set_error(TQ_ERR_VALUE, "head_dim must be 64 or 128");
  if (out_dtype != TQ_BF16 && out_dtype != TQ_F32) return set_error(TQ_ERR_VALUE, "out_dtype must be BF16 or F32");
  if (num_seqs == 0) return TQ_OK;
  if (!part_out || !part_lse || !out) return set_error(TQ_ERR_VALUE, "NULL merge buffer");
  MergeParams mp = {part_out, part_lse, out, lse, num_seqs, num_heads, num_splits, head_dim, out_dtype == TQ_F32, 0};
  launch_merge(mp, (int64_t)num_seqs * num_heads, reinterpret_cast<hipStream_t>(stream));
  return launch_status("tq_split_merge launch");
}

namespace {
// A dense window attended with the history (tq_decode_paged_window).
struct WinArgs {
  const void* k;
  const void* v;
  int32_t capacity;
  const int32_t* lens;
};

tq_status decode_impl(const void* q, tq_dtype q_dtype, int32_t num_seqs, int32_t num_queries,
                      int32_t num_q_heads, int32_t num_kv_heads, const uint8_t* k_pages,
                      const uint8_t* v_pages, int64_t num_blocks, int32_t block_size,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, const tq_format* kfmt, const tq_format* vfmt,
                      float scale, int32_t num_splits, void* workspace, uint64_t workspace_bytes,
                      void* out, tq_dtype out_dtype, float* lse, int32_t* dev_err,
                      tq_stream_t stream, const WinArgs* win) {
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
  if (num_queries <= 0) return set_error(TQ_ERR_VALUE, "num_queries must be >= 1");
  if (!(scale > 0.f) || !(scale < INFINITY)) return set_error(TQ_ERR_VALUE, "scale must be positive and finite");
  if (block_size != TQ_BLOCK_SIZE) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "block_size must be 16");
  const int Gr = num_q_heads / num_kv_heads;
  if ((int64_t)num_queries * Gr > TQ_MAX_COLUMNS)
    return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "more than " + std::to_string(TQ_MAX_COLUMNS) +
                                                    " (query, q head) pairs per kv head");
  const int G = num_queries * Gr;   // matrix-core columns used per kv head
  const int kk = format_kind_k(kfmt), vk = format_kind_v(vfmt);
  if (vfmt->qjl) return set_error(TQ_ERR_VALUE, "the QJL stage is defined for K formats only");
  // QJL formats whose MSE groups and V format the main kernel reads take it
  // (the sketch term on the matrix cores, up to 64 columns per kv head);
  // other QJL layouts take the separate QJL kernel (one query, <= 8 q heads)
  const bool qjl_fast = kfmt->qjl && kk >= 0 && (vk == V4 || vk == V2);
  if (qjl_fast && G > 64)
    return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "K formats with the QJL stage take at most 64 (query, q head) pairs per kv head");
  if (kfmt->qjl && !qjl_fast && num_queries != 1)
    return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "this QJL K format takes one query per sequence");
  if (kfmt->qjl && !qjl_fast && Gr > 8)
    return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "this QJL K format takes at most 8 q heads per kv head");
  if (kk < 0 && !kfmt->qjl) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "no decode kernel for this K format (served: 4-bit, 2-bit, 4+3-bit and 3+2-bit groups)");
  if (vk < 0)
    return set_error(TQ_ERR_UNSUPPORTED_FORMAT,
                     "no decode kernel for this V format (served: 4-bit, 2-bit, 4+3-bit and 3+2-bit groups)");
  if (kfmt->qjl && (vk == VM43 || vk == VM32))
    return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "K formats with the QJL stage take one-group V formats");
  const int D = kfmt->head_dim;
  if (num_seqs == 0) return TQ_OK;
  if (!q || !k_pages || !v_pages || !block_tables || !context_lens || !out)
    return set_error(TQ_ERR_VALUE, "NULL required pointer");
  if (win) {   // the window's result takes one more partial slot per row
    if (num_queries != 1) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "a dense window takes one query per sequence");
    if (Gr > 16) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "a dense window takes at most 16 q heads per kv head");
    if (kfmt->qjl && !qjl_fast) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "this QJL K format takes no dense window");
    if (win->capacity < 0) return set_error(TQ_ERR_VALUE, "window capacity must be >= 0");
    if (num_seqs > 0 && !win->lens) return set_error(TQ_ERR_VALUE, "NULL window lengths");
    if (win->capacity > 0 && (!win->k || !win->v)) return set_error(TQ_ERR_VALUE, "NULL window K or V");
    if ((reinterpret_cast<uintptr_t>(win->k) | reinterpret_cast<uintptr_t>(win->v)) & 15u)
      return set_error(TQ_ERR_VALUE, "window K and V must be 16-byte aligned");
    if ((int64_t)num_seqs * win->capacity * num_kv_heads * D * 2 >= (1ll << 40))
      return set_error(TQ_ERR_VALUE, "window too large");
  }
  const int slots = num_splits + (win ? 1 : 0);   // partial slots per row
  uint64_t need = 0;
  tq_decode_workspace_bytes(num_seqs * num_queries, num_q_heads, D, win ? slots : num_splits, &need);
  if (workspace_bytes < need || (need && !workspace))
    return set_error(TQ_ERR_VALUE, "workspace too small: need " + std::to_string(need) + " bytes");
  const int64_t work_bound = (int64_t)num_seqs * num_kv_heads * (max_blocks_per_seq + 128);
  if (work_bound >= (1ll << 30) || max_blocks_per_seq > (1 << 20))
    return set_error(TQ_ERR_VALUE, "too much work for one call (2^30 block-heads, 2^20 blocks per sequence)");
  const int64_t q_bytes = (int64_t)num_seqs * num_queries * num_q_heads * D * (q_dtype == TQ_F32 ? 4 : 2);
  const int64_t k_pool = num_blocks * num_kv_heads * (int64_t)tile_bytes_of(kfmt);
  const int64_t v_pool = num_blocks * num_kv_heads * (int64_t)tile_bytes_of(vfmt);
  if (num_blocks >= (1ll << 31) || k_pool > 0xFFFFFFFFll || v_pool > 0xFFFFFFFFll)
    return set_error(TQ_ERR_VALUE, "each page pool must be smaller than 4 GiB");
  if (q_bytes >= (1ll << 31)) return set_error(TQ_ERR_VALUE, "q must be smaller than 2 GiB");
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);

  if (kfmt->qjl && (reinterpret_cast<uintptr_t>(kfmt->qjl_proj) & 15))
    return set_error(TQ_ERR_VALUE, "qjl_proj must be 16-byte aligned");
  if (kfmt->qjl && !qjl_fast) {   // sketch term on every score: the QJL decode kernel, then the generic merge
    if ((reinterpret_cast<uintptr_t>(k_pages) | reinterpret_cast<uintptr_t>(v_pages) |
         reinterpret_cast<uintptr_t>(kfmt->qjl_proj)) & 15)
      return set_error(TQ_ERR_VALUE, "page pools and qjl_proj must be 16-byte aligned");
    DevFormat kf, vf;
    make_dev_format(kfmt, &kf);
    make_dev_format(vfmt, &vf);
    if (vf.row_bytes % 16 == 0) vf.chunk = vf.row_bytes / 16;   // lane-major V index plane
    QjlDecodeArgs qa = {};
    qa.q = q;
    qa.q_f32 = q_dtype == TQ_F32;
    qa.S = num_seqs;
    qa.Hq = num_q_heads;
    qa.Hkv = num_kv_heads;
    qa.G = Gr;
    qa.k_pages = k_pages;
    qa.v_pages = v_pages;
    qa.num_blocks = num_blocks;
    qa.block_tables = block_tables;
    qa.max_blocks = max_blocks_per_seq;
    qa.context_lens = context_lens;
    qa.proj = kfmt->qjl_proj;
    qa.scale = scale;
    qa.P = num_splits;
    qa.out = out;
    qa.out_f32 = out_dtype == TQ_F32;
    qa.lse = lse;
    qa.dev_err = dev_err;
    if (num_splits > 1) {
      qa.part_o = static_cast<float*>(workspace);
      qa.part_lse = qa.part_o + (int64_t)num_seqs * num_q_heads * num_splits * D;
    }
    st = launch_qjl_decode(qa, kf, vf, hs);
    if (st != TQ_OK || num_splits == 1) return st;
    MergeParams mp = {qa.part_o, qa.part_lse, out, lse, num_seqs, num_q_heads, num_splits, D, qa.out_f32, 0};
    launch_merge(mp, (int64_t)num_seqs * num_q_heads, hs);
    return launch_status("tq_decode_paged merge launch");
  }

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
  // One 16-wave workgroup per CU.  The G columns of a kv head are taken in
  // CG groups of 8 (CG the power of two with 8 CG >= G).  A workgroup takes
  // the HG kv heads of a group together (its waves read the HG adjacent
  // tiles of each physical block); HG is the largest of 8, 4, 2, 1 dividing
  // Hkv with HG * CG <= 16 that still leaves at least one piece per CU when
  // every context is full length.
  int CG = 1;
  while (8 * CG < G) CG *= 2;
  const int cus = device_cus();
  int HG = 1;
  const int vh_cap = qjl_fast ? 8 : 16;   // QJL: the sketch operands take the other 8 operand areas
  for (int hg : {8, 4, 2}) {
    if (num_kv_heads % hg || hg * CG > vh_cap) continue;
    if ((int64_t)num_seqs * (num_kv_heads / hg) * num_splits >= cus) { HG = hg; break; }
  }
  p.HG = HG;
  p.NG = num_kv_heads / HG;
  p.CG = CG;
  p.VH = HG * CG;
  // starting a piece (set-up, rotation of q, epilogue) costs about as much
  // time as streaming 128 tiles of one kv head for one column group, i.e.
  // 128 / (HG CG) blocks
  p.seg_cost = 128 / (HG * CG);
  p.inv_G = 1.0f / (float)G;
  p.NQ = num_queries;
  p.Gr = Gr;
  p.rows_ps = num_queries * num_q_heads;
  p.inv_Gr = 1.0f / (float)Gr;
  p.win_items = win ? num_seqs * num_kv_heads : 0;
  const int64_t units = (int64_t)num_seqs * p.NG * max_blocks_per_seq;
  p.n_wg = (int)(units < cus ? (units > 0 ? units : 1) : cus);
  p.k_tile = tile_bytes_of(kfmt);
  p.v_tile = tile_bytes_of(vfmt);
  p.k_span = (uint32_t)k_pool;
  p.v_span = (uint32_t)v_pool;
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
  // LUT halves: K's 4-bit or 2-bit table in half 0 (the 2-bit group's for
  // 3+2 bits); V's 4-bit or 2-bit group shares it when bits and codebook
  // agree, else takes half 1.  The 3-bit groups (K's and V's) share the pair
  // table, so their levels must agree.
  const int kgh = kk == KM32 ? 1 : 0;   // K group whose levels fill half 0
  const int kbits0 = kfmt->group_bits[kgh];
  p.half_kind[0] = kbits0;
  for (int i = 0; i < 16; ++i) p.half_cb[0][i] = kfmt->codebook[kgh][i];
  const int vgh = vk == VM32 ? 1 : 0;   // V group read through a LUT half
  const int vbits = vfmt->group_bits[vgh];
  bool share = vbits == kbits0;
  for (int i = 0; i < (1 << vbits) && share; ++i) share = vfmt->codebook[vgh][i] == kfmt->codebook[kgh][i];
  if (share) {
    p.v_half = 0;
    p.half_kind[1] = 0;
  } else {
    p.v_half = 1;
    p.half_kind[1] = vbits;
    for (int i = 0; i < 16; ++i) p.half_cb[1][i] = vfmt->codebook[vgh][i];
  }
  const bool kmix = kk == KM43 || kk == KM32, vmix = vk == VM43 || vk == VM32;
  if (kmix)   // the 3-bit group's levels: group 1 (4+3) or group 0 (3+2)
    for (int i = 0; i < 8; ++i) p.k3_cb[i] = kfmt->codebook[kk == KM43 ? 1 : 0][i];
  if (vmix) {
    const uint16_t* v3 = vfmt->codebook[vk == VM43 ? 1 : 0];
    for (int i = 0; i < 8; ++i) {
      if (kmix && p.k3_cb[i] != v3[i])
        return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "K and V 3-bit groups with different codebooks");
      p.k3_cb[i] = v3[i];
    }
    for (int jx = 0; jx < D; ++jx) p.v_ch[jx] = vfmt->group_channels[jx];
  }
  p.proj = kfmt->qjl_proj;
  p.q_f32 = q_dtype == TQ_F32;
  p.out_f32 = out_dtype == TQ_F32;
  p.q_bytes = (int32_t)q_bytes;
#ifdef TQ_PHASE_TRACE
  p.trace = __atomic_load_n(&g_phase_trace, __ATOMIC_ACQUIRE);
#endif
  p.PS = slots;
  if (win) {
    p.win_on = 1;
    p.win_k = win->k;
    p.win_v = win->v;
    p.win_lens = win->lens;
    p.win_cap = win->capacity;
    p.win_scale_log2 = (float)((double)scale * 1.4426950408889634);
  }
  if (slots > 1) {
    p.part_o = static_cast<float*>(workspace);
    p.part_lse = p.part_o + (int64_t)num_seqs * num_queries * num_q_heads * slots * D;
  }
  const int kk_launch = kk | (qjl_fast ? KQ : 0);   // K kind with the QJL flag
#define TQ_LAUNCH(DD, KKK, VVV) \
  if (D == DD && kk_launch == (KKK) && vk == VVV) launch_decode<DD, (KKK), VVV>(p, hs);
#define TQ_LAUNCH_V(DD, KKK) TQ_LAUNCH(DD, KKK, V4) TQ_LAUNCH(DD, KKK, V2) TQ_LAUNCH(DD, KKK, VM43) TQ_LAUNCH(DD, KKK, VM32)
#define TQ_LAUNCH_Q(DD, KKK) TQ_LAUNCH(DD, KKK | KQ, V4) TQ_LAUNCH(DD, KKK | KQ, V2)
  TQ_LAUNCH_V(128, K4) TQ_LAUNCH_V(128, K2) TQ_LAUNCH_V(128, KM43) TQ_LAUNCH_V(128, KM32)
  TQ_LAUNCH_V(64, K4) TQ_LAUNCH_V(64, K2) TQ_LAUNCH_V(64, KM43) TQ_LAUNCH_V(64, KM32)
  TQ_LAUNCH_Q(128, K4) TQ_LAUNCH_Q(128, K2) TQ_LAUNCH_Q(128, KM43) TQ_LAUNCH_Q(128, KM32)
  TQ_LAUNCH_Q(64, K4) TQ_LAUNCH_Q(64, K2) TQ_LAUNCH_Q(64, KM43) TQ_LAUNCH_Q(64, KM32)
#undef TQ_LAUNCH_Q
#undef TQ_LAUNCH_V
#undef TQ_LAUNCH
  st = launch_status("tq_decode_paged launch");
  if (st != TQ_OK || slots == 1) return st;
  MergeParams mp = {p.part_o, p.part_lse, out, lse, num_seqs * num_queries, num_q_heads, slots, D,
                    p.out_f32, 1};
  launch_merge(mp, (int64_t)num_seqs * num_queries * num_q_heads, hs);
  return launch_status("tq_decode_paged merge launch");
}
}  // namespace

extern "C" tq_status tq_decode_paged_multi(const void* q, tq_dtype q_dtype, int32_t num_seqs, int32_t num_queries,
                                           int32_t num_q_heads, int32_t num_kv_heads, const uint8_t* k_pages,
                                           const uint8_t* v_pages, int64_t num_blocks, int32_t block_size,
                                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, const tq_format* kfmt, const tq_format* vfmt,
                                           float scale, int32_t num_splits, void* workspace, uint64_t workspace_bytes,
                                           void* out, tq_dtype out_dtype, float* lse, int32_t* dev_err,
                                           tq_stream_t stream) {
  return decode_impl(q, q_dtype, num_seqs, num_queries, num_q_heads, num_kv_heads, k_pages, v_pages, num_blocks,
                     block_size, block_tables, max_blocks_per_seq, context_lens, kfmt, vfmt, scale, num_splits,
                     workspace, workspace_bytes, out, out_dtype, lse, dev_err, stream, nullptr);
}

extern "C" tq_status tq_decode_paged_window(const void* q, tq_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, const uint8_t* k_pages, const uint8_t* v_pages,
                                            int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
                                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                                            const tq_format* kfmt, const tq_format* vfmt, const void* win_k,
                                            const void* win_v, tq_dtype win_dtype, int32_t win_capacity,
                                            const int32_t* win_lens, float scale, int32_t num_splits,
                                            void* workspace, uint64_t workspace_bytes, void* out, tq_dtype out_dtype,
                                            float* lse, int32_t* dev_err, tq_stream_t stream) {
  if (win_dtype != TQ_BF16)
    return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "the fused window takes bf16 rows (use tq_decode_dense for f32)");
  const WinArgs win = {win_k, win_v, win_capacity, win_lens};
  return decode_impl(q, q_dtype, num_seqs, 1, num_q_heads, num_kv_heads, k_pages, v_pages, num_blocks, block_size,
                     block_tables, max_blocks_per_seq, context_lens, kfmt, vfmt, scale, num_splits, workspace,
                     workspace_bytes, out, out_dtype, lse, dev_err, stream, &win);
}

// ------------------------------------------------------------ no allocation
// Split workspace of tq_decode_paged_noalloc: one array per GPU, part of the
// library's code object, held until the process ends.  Host code must not
// pass the array's name to a kernel (in host code it names a host-side
// stand-in); its device address is looked up once per device below.
static __device__ __align__(256) uint8_t scratch[TQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on each device, with that device current).
tq_status scratch_address(void** out) {
  int dev = -1;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) return set_error(TQ_ERR_DEVICE, std::string("hipGetDevice: ") + hipGetErrorString(ge));
  if (dev < 0 || dev >= kMaxDevices) return set_error(TQ_ERR_DEVICE, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return set_error(TQ_ERR_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TQ_OK;
}
}  // namespace

extern "C" tq_status tq_decode_paged_noalloc(const void* q, tq_dtype q_dtype, int32_t num_seqs,
                                             int32_t num_q_heads, int32_t num_kv_heads, const uint8_t* k_pages,
                                             const uint8_t* v_pages, int64_t num_blocks, int32_t block_size,
                                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                                             const int32_t* context_lens, const tq_format* kfmt,
                                             const tq_format* vfmt, float scale, int32_t num_splits, void* out,
                                             tq_dtype out_dtype, float* lse, int32_t* dev_err, tq_stream_t stream) {
  if (!kfmt) return set_error(TQ_ERR_VALUE, "NULL format");
  uint64_t need = 0;
  tq_status st = tq_decode_workspace_bytes(num_seqs, num_q_heads, kfmt->head_dim, num_splits, &need);
  if (st != TQ_OK) return st;
  if (need > TQ_NOALLOC_SCRATCH_BYTES)
    return set_error(TQ_ERR_VALUE, "split workspace of " + std::to_string(need) + " bytes exceeds the " +
                                       std::to_string((unsigned long long)TQ_NOALLOC_SCRATCH_BYTES) +
                                       " bytes the allocation-free call holds per GPU (use fewer splits, or "
                                       "tq_decode_paged with a workspace)");
  void* ws = nullptr;
  if (need) {
    st = scratch_address(&ws);
    if (st != TQ_OK) return st;
  }
  return tq_decode_paged_multi(q, q_dtype, num_seqs, 1, num_q_heads, num_kv_heads, k_pages, v_pages, num_blocks,
                               block_size, block_tables, max_blocks_per_seq, context_lens, kfmt, vfmt, scale,
                               num_splits, ws, need ? TQ_NOALLOC_SCRATCH_BYTES : 0, out, out_dtype, lse, dev_err,
                               stream);
}

extern "C" tq_status tq_decode_paged(const void* q, tq_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t num_kv_heads, const uint8_t* k_pages, const uint8_t* v_pages,
                                     int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                                     const tq_format* kfmt, const tq_format* vfmt, float scale,
                                     int32_t num_splits, void* workspace, uint64_t workspace_bytes, void* out,
                                     tq_dtype out_dtype, float* lse, int32_t* dev_err, tq_stream_t stream) {
  return tq_decode_paged_multi(q, q_dtype, num_seqs, 1, num_q_heads, num_kv_heads, k_pages, v_pages, num_blocks,
                               block_size, block_tables, max_blocks_per_seq, context_lens, kfmt, vfmt, scale,
                               num_splits, workspace, workspace_bytes, out, out_dtype, lse, dev_err, stream);
}
