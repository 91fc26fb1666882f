// Host side of libtq: status and error messages, format validation, byte
// math, and the Lloyd-Max codebook solver.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "tq_internal.h"

namespace tq {

static thread_local std::string g_last_error;

tq_status set_error(tq_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

tq_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    return set_error(TQ_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
  }
  return TQ_OK;
}

// [D "Error Model"]: bad shapes, unsupported bit widths and malformed
// metadata are value errors; [D "Recipe Strategy"]: the runtime validates
// head dimension and group sizes of the metadata it loads.
tq_status check_format(const tq_format* f, const char* which) {
  std::string w(which);
  if (!f) return set_error(TQ_ERR_VALUE, w + " format is NULL");
  if (f->head_dim != 64 && f->head_dim != 128)
    return set_error(TQ_ERR_VALUE, w + " head_dim must be 64 or 128");
  if (f->num_groups != 1 && f->num_groups != 2)
    return set_error(TQ_ERR_VALUE, w + " num_groups must be 1 or 2");
  const int d = f->head_dim, m = d / f->num_groups;
  bool seen[TQ_MAX_HEAD_DIM] = {false};
  for (int j = 0; j < d; ++j) {
    const int c = f->group_channels[j];
    if (c >= d || seen[c]) return set_error(TQ_ERR_VALUE, w + " group_channels is not a permutation of 0..d-1");
    seen[c] = true;
    if (j % m != 0 && f->group_channels[j] <= f->group_channels[j - 1])
      return set_error(TQ_ERR_VALUE, w + " group_channels must ascend within each group");
    if (f->num_groups == 1 && c != j)
      return set_error(TQ_ERR_VALUE, w + " a single group lists channels in natural order");
    if (f->signs[j] != 1 && f->signs[j] != -1) return set_error(TQ_ERR_VALUE, w + " signs must be +1 or -1");
  }
  for (int g = 0; g < f->num_groups; ++g) {
    const int b = f->group_bits[g];
    if (b < 2 || b > 4) return set_error(TQ_ERR_VALUE, w + " group_bits must be 2, 3 or 4");
    double prev = -INFINITY;
    for (int i = 0; i < (1 << b); ++i) {
      const uint16_t h = f->codebook[g][i];
      if ((h & 0x7C00u) == 0x7C00u) return set_error(TQ_ERR_VALUE, w + " codebook entries must be finite");
      const double v = f16_bits_to_f64(h);
      if (!(v > prev)) return set_error(TQ_ERR_VALUE, w + " codebook must be strictly ascending");
      prev = v;
    }
  }
  if (f->qjl != 0 && f->qjl != 1) return set_error(TQ_ERR_VALUE, w + " qjl must be 0 or 1");
  if (f->qjl && !f->qjl_proj) return set_error(TQ_ERR_VALUE, w + " qjl_proj is NULL");
  return TQ_OK;
}

int mse_row_bytes(const tq_format* f) {
  const int m = f->head_dim / f->num_groups;
  int bits = 0;
  for (int g = 0; g < f->num_groups; ++g) bits += m * f->group_bits[g];
  return bits / 8;
}

int row_index_bytes(const tq_format* f) { return mse_row_bytes(f) + (f->qjl ? f->head_dim / 8 : 0); }

int tile_bytes_of(const tq_format* f) {
  const int raw = TQ_BLOCK_SIZE * row_index_bytes(f) + TQ_BLOCK_SIZE * f->num_groups * 2 * (f->qjl ? 2 : 1);
  return (raw + 15) / 16 * 16;
}

void make_dev_format(const tq_format* f, DevFormat* o) {
  memset(o, 0, sizeof(*o));
  o->d = f->head_dim;
  o->ng = f->num_groups;
  o->m = f->head_dim / f->num_groups;
  for (int j = 0; j < f->head_dim; ++j) {
    if (f->signs[j] < 0) o->sign_bits[j >> 5] |= 1u << (j & 31);
    o->ch[j] = f->group_channels[j];
  }
  int off = 0;
  for (int g = 0; g < f->num_groups; ++g) {
    o->bits[g] = f->group_bits[g];
    o->grp_byte_off[g] = off;
    off += o->m * f->group_bits[g] / 8;
    for (int i = 0; i < 16; ++i) o->cb[g][i] = f->codebook[g][i];
    for (int i = 0; i + 1 < (1 << f->group_bits[g]); ++i)   // exact in fp64
      o->thr[g][i] = (f16_bits_to_f64(f->codebook[g][i]) + f16_bits_to_f64(f->codebook[g][i + 1])) * 0.5;
    const int nthr = (1 << f->group_bits[g]) - 1;
    for (double off : {128.5, 128.25, 128.75, 128.375, 128.625, 128.125, 128.875}) {
      bool ok = true;
      double prev = -1.0;
      for (int i = 0; i < nthr && ok; ++i) {
        const double x = o->thr[g][i] * 32.0 + off;
        const double b = floor(x), fr = x - b;
        ok = x >= 1.0 && x < 255.0 && fr >= 0.02 && fr <= 0.98 && b > prev;
        prev = b;
      }
      if (ok) {
        o->lut_off[g] = (float)off;
        o->fast[g] = 1;
        break;
      }
    }
  }
  o->row_bytes = row_index_bytes(f);
  o->tile_bytes = tile_bytes_of(f);
  o->norm_off = TQ_BLOCK_SIZE * o->row_bytes;
  o->qjl = f->qjl;
  o->sign_off = mse_row_bytes(f);
  o->rnorm_off = o->norm_off + TQ_BLOCK_SIZE * f->num_groups * 2;
}

// ------------------------------------------------------------ Lloyd-Max
// Max's construction for a symmetric unit Gaussian: guess the first
// positive level y1, then march outwards -- each cell's far edge is where
// the cell's conditional mean equals its level, and the next level mirrors
// the current one about that edge -- and adjust y1 by bisection until the
// outermost level is the conditional mean of the unbounded last cell.
// Extended precision (long double) throughout; the caller rounds to fp16.

static long double pdf(long double x) { return expl(-0.5L * x * x) * 0.39894228040143267793994605993438L; }

// P(a < X < b) for 0 <= a < b (b may be +inf), via complementary erf.
static long double prob_pos(long double a, long double b) {
  const long double r2 = 0.70710678118654752440084436210485L;
  const long double qa = 0.5L * erfcl(a * r2);
  const long double qb = isinf(b) ? 0.0L : 0.5L * erfcl(b * r2);
  return qa - qb;
}

static long double cell_mean(long double a, long double b) {
  const long double pb = isinf(b) ? 0.0L : pdf(b);
  return (pdf(a) - pb) / prob_pos(a, b);
}

// Edge x > a with cell_mean(a, x) == y; returns +inf if even the unbounded
// cell's mean is below y (the guess was too large).
static long double edge_for_mean(long double a, long double y) {
  if (cell_mean(a, INFINITY) <= y) return INFINITY;
  long double lo = a, hi = a + 1.0L;
  while (cell_mean(a, hi) < y) hi = a + 2.0L * (hi - a);
  for (int it = 0; it < 200; ++it) {
    const long double mid = 0.5L * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (cell_mean(a, mid) < y) lo = mid; else hi = mid;
  }
  return 0.5L * (lo + hi);
}

// Shooting residual for a first level y1 (positive half of `half` levels).
// Returns > 0 when y1 is too large.
static long double shoot(long double y1, int half, long double* levels) {
  long double a = 0.0L, y = y1;
  for (int i = 0; i < half - 1; ++i) {
    levels[i] = y;
    const long double x = edge_for_mean(a, y);
    if (isinf(x)) return 1.0L;
    const long double yn = 2.0L * x - y;
    if (!(yn > y)) return 1.0L;
    a = x;
    y = yn;
  }
  levels[half - 1] = y;
  return y - cell_mean(a, INFINITY);
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::mutex mu;
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace tq

using namespace tq;

extern "C" {

const char* tq_last_error(void) { return g_last_error.c_str(); }

tq_status tq_lloyd_max_codebook(int32_t bits, uint16_t* out) {
  if (!out) return set_error(TQ_ERR_VALUE, "output pointer is NULL");
  if (bits < 1 || bits > 4) return set_error(TQ_ERR_VALUE, "bits must be in 1..4");
  const int L = 1 << bits, half = L / 2;
  long double levels[8];
  long double lo = 0.0L, hi = 0.7978845608028653558798921198687637L;  // y1 < E|X|
  if (half == 1) {
    levels[0] = cell_mean(0.0L, INFINITY);
  } else {
    for (int it = 0; it < 200; ++it) {
      const long double mid = 0.5L * (lo + hi);
      if (mid == lo || mid == hi) break;
      if (shoot(mid, half, levels) > 0) hi = mid; else lo = mid;
    }
    shoot(0.5L * (lo + hi), half, levels);
  }
  for (int i = 0; i < half; ++i) {
    const uint16_t p = f64_to_f16_rne((double)levels[i]);
    out[half + i] = p;
    out[half - 1 - i] = (uint16_t)(p | 0x8000u);
  }
  g_last_error.clear();
  return TQ_OK;
}

tq_status tq_format_check(const tq_format* f) { return check_format(f, "format"); }

tq_status tq_tile_bytes(const tq_format* f, int32_t block_size, int32_t* rib, int32_t* tb) {
  tq_status st = check_format(f, "format");
  if (st != TQ_OK) return st;
  if (!rib || !tb) return set_error(TQ_ERR_VALUE, "output pointer is NULL");
  if (block_size != TQ_BLOCK_SIZE) return set_error(TQ_ERR_UNSUPPORTED_FORMAT, "block_size must be 16");
  *rib = row_index_bytes(f);
  *tb = tile_bytes_of(f);
  return TQ_OK;
}

tq_status tq_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                    int32_t num_splits, uint64_t* bytes) {
  if (!bytes) return set_error(TQ_ERR_VALUE, "output pointer is NULL");
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits <= 0)
    return set_error(TQ_ERR_VALUE, "shape arguments must be positive");
  *bytes = num_splits > 1 ? (uint64_t)num_seqs * num_q_heads * num_splits * (head_dim + 1) * 4ull : 0ull;
  return TQ_OK;
}

}  // extern "C"
