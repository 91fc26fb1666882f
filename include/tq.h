/*
 * tq.h -- C ABI of libtq: quantise-on-write into packed KV pages and paged
 * decode attention that consumes the packed pages directly (MI355X, gfx950).
 *
 * The method: each cached K or V row is rotated (seeded +-1 signs, then a
 * Walsh-Hadamard transform scaled by 1/sqrt(d)), split into one or two
 * channel groups, each group stored as an fp16 vector norm plus per-channel
 * indices into a Lloyd-Max codebook, packed LSB-first into uint8 pages.
 *
 * Sources, cited by page title and section:
 *   [D] TurboQuant documentation, "Design" page: "System Invariants",
 *       "Data Ownership", "Serving Route Design", "Format Strategy",
 *       "Recipe Strategy", "Error Model".
 *   [S] "TurboQuant Inference Server" README: "What it does",
 *       "Architecture notes" (Lloyd-Max codebooks computed once on the CPU).
 *   [T] "Tattletale" README, "Highlights" (random Hadamard rotation plus
 *       codebooks).
 *
 * Ownership and threading ([D "Data Ownership"]: the cache owner owns the
 * persistent bytes, the attention path only consumes them):
 *   - The caller allocates every buffer (pages, q, out, lse, workspace,
 *     slot_mapping, block tables, context lengths, error words).  The library
 *     allocates nothing; its only state between calls is the device array of
 *     tq_decode_paged_noalloc (part of its code object, one per GPU).
 *   - Pointers named "device" must be device memory; "host" pointers are
 *     read during the call only.
 *   - Every GPU call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream).  Buffers must stay valid until that work completes.
 *   - Page pools are never cleared by the library; bytes of rows that were
 *     never written are unspecified.
 *   - Calls are thread-safe; tq_last_error() is per thread.
 *
 * Errors ([D "Error Model"]; a Python binding maps them to exceptions):
 *   TQ_ERR_VALUE        bad shapes, dtypes, bit widths, group sizes,
 *                       malformed codebook / signs / channel list, NULL
 *                       required pointer, workspace too small  (ValueError)
 *   TQ_ERR_INDEX        slot or block-table entry outside the pool; for
 *                       device-resident data this is reported through the
 *                       optional device error word        (IndexError)
 *   TQ_ERR_UNSUPPORTED_FORMAT  a valid format no kernel serves; the library
 *                       never falls back to a dense path
 *                       ([D "System Invariants", "Serving Route Design"])
 *   TQ_ERR_NOT_FOUND    reserved for metadata loaders   (FileNotFoundError)
 *   TQ_ERR_DEVICE       HIP launch or runtime failure
 *
 * Device error word: `int32_t dev_err[2]` in device memory, zeroed by the
 * caller.  A kernel that meets an out-of-range slot or block-table entry
 * sets dev_err[0] = TQ_ERR_INDEX (if it was 0) and dev_err[1] = the position
 * of that entry (see each call); which entry is recorded when several are
 * bad is unspecified.  The offending row is not written / the offending
 * block is skipped; nothing is read or written out of bounds.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* tq_stream_t; /* same type as hipStream_t */

typedef enum tq_status {
  TQ_OK = 0,
  TQ_ERR_VALUE = 1,
  TQ_ERR_INDEX = 2,
  TQ_ERR_UNSUPPORTED_FORMAT = 3,
  TQ_ERR_NOT_FOUND = 4,
  TQ_ERR_DEVICE = 5
} tq_status;

/* The two bounding enumerators give the type the range of int32, so that
 * any int32 a caller passes as a dtype is a value of the type (and is
 * rejected by the calls' checks unless it is TQ_F32 or TQ_BF16). */
typedef enum tq_dtype {
  TQ_F32 = 0,
  TQ_BF16 = 1,
  TQ_DTYPE_RANGE_LOW_ = -2147483647 - 1,
  TQ_DTYPE_RANGE_HIGH_ = 2147483647
} tq_dtype;

#define TQ_MAX_HEAD_DIM 128
#define TQ_BLOCK_SIZE 16
/* (query, q head) pairs a paged decode call serves per kv head */
#define TQ_MAX_COLUMNS 128

/*
 * One tensor's storage format.  K and V each get their own, chosen
 * independently of each other ([D "System Invariants"]).  Host struct,
 * read during the call.
 *
 *   head_dim        64 or 128.
 *   num_groups      1 or 2.  Two groups split the rotated channels into a
 *                   high-precision and a low-precision half, chosen by
 *                   metadata, never guessed at run time ([D "Recipe
 *                   Strategy"]).  Each group has head_dim / num_groups
 *                   channels.
 *   group_bits      bits per index of each group: 2, 3 or 4.
 *   group_channels  rotated-domain channel ids: group 0 ascending, then
 *                   group 1 ascending (a permutation of 0..head_dim-1); the
 *                   identity for one group.
 *   codebook        per group, 2^bits fp16 bit patterns: finite, strictly
 *                   ascending unit-variance levels (entries beyond 2^bits
 *                   are ignored).  tq_lloyd_max_codebook() fills them.
 *   signs           +1 / -1 per channel: the seeded signs of the rotation.
 *   qjl             0, or 1 for a K format whose groups also store the QJL
 *                   residual stage ([D "Recipe Strategy"]: each group stores
 *                   [MSE indices][QJL signs][vector norm][residual norm];
 *                   the pages define only the field names, the stage below
 *                   is the published quantised Johnson-Lindenstrauss
 *                   transform).  V formats must have qjl = 0.
 *   qjl_proj        qjl = 1: DEVICE pointer to the projections, fp32
 *                   [num_groups][m][m] row-major (entry [g][i][j] multiplies
 *                   residual channel j of group g into output i), i.i.d.
 *                   N(0, 1) values drawn by the caller, 16-byte aligned;
 *                   read by tq_write_kv and tq_decode_paged during the call.
 *                   Unused when qjl = 0.
 *
 * Encoding of a row x (head_dim values), per group G of m channels:
 *   w   = H (signs * x)           Sylvester Walsh-Hadamard, natural order,
 *                                 fp64 butterflies h = 1, 2, ..., d/2
 *   ss  = pairwise-tree sum of w_j^2 over G (adjacent pairs first), fp64
 *   norm= fp16 round-to-nearest-even of sqrt(ss / head_dim)
 *   T_i = fp64 (t_i * sqrt(ss / m)), t_i = midpoint of levels i, i+1
 *   idx = number of thresholds T_i strictly below w_j
 *   (ss == 0: norm +0 and every index 2^bits/2 - 1)
 * Decoding: rotated value of channel j in G is norm * codebook[idx] / sqrt(m).
 *
 * QJL stage (qjl = 1), per group G after the above, fp64, no fused
 * multiply-add:
 *   a     = norm (the stored fp16 value) * sqrt(head_dim / m)
 *   r_j   = w_j - a * codebook[idx_j]                 residual, j in G
 *   rnorm = fp16 RNE of sqrt(pairwise-tree sum of r_j^2 / head_dim)
 *   z_i   = sum_j proj[g][i][j] * r_j, evaluated from +0 over j ascending,
 *           each product and then each partial sum rounded to fp64 (never
 *           fused); sign bit i = (z_i < 0)
 * Decoding adds, per group, sqrt(pi/2) / m * rnorm * sum_i (P_g q~_G)_i
 * (1 - 2 bit_i) to the rotated score q~ . k (q~ the rotated, normalised
 * query restricted to G): an unbiased estimate of q~ . (y_G - y_hat_G).
 * The fixed order makes every sign bit well defined, also for a z_i whose
 * exact value lies within rounding of zero.
 */
typedef struct tq_format {
  int32_t head_dim;
  int32_t num_groups;
  int32_t group_bits[2];
  uint8_t group_channels[TQ_MAX_HEAD_DIM];
  uint16_t codebook[2][16];
  int8_t signs[TQ_MAX_HEAD_DIM];
  int32_t qjl;
  const float* qjl_proj;
} tq_format;

/*
 * Page layout ([D "Serving Route Design"]: slot -> physical block -> token
 * offset -> packed row bytes, with block = slot / 16 and offset = slot % 16):
 *   pages  : [num_blocks][num_kv_heads][tile_bytes] uint8, device memory.
 *   tile   : index plane of 16 packed rows (each group's indices packed
 *            LSB-first, group 0 first, row_index_bytes per row), then the
 *            norm plane: fp16 little-endian, group-major, the norm of group g
 *            of the row at in-block offset t stored at
 *            16*row_index_bytes + 2*(16*g + 4*(t % 4) + t / 4).
 *            The tile is padded to a multiple of 16 bytes.
 *   QJL K formats: a row's index bytes are its MSE indices followed by its
 *            sign bits (head_dim / 8 bytes: group 0's m bits, then group
 *            1's, output i of a group at bit i, LSB-first); the norm plane
 *            holds the vector norms as above, then the residual norms in the
 *            same arrangement (residual norm of group g at norm plane slot
 *            16*(num_groups + g) + 4*(t % 4) + t / 4).
 *   index plane, K pages: row t at bytes [t*rb, (t+1)*rb), rb = row_index_bytes.
 *   index plane, V pages: when rb is a multiple of 16 (c = rb / 16), byte b
 *            of row t is at ((16*(t % 4) + b / c)*4 + t / 4)*c + b % c: 64 runs
 *            of 4c bytes, run 16q + j holding bytes [c*j, c*(j+1)) of rows q,
 *            q+4, q+8, q+12 (one decode lane's share, one wide load).
 *            Two-group V formats: group g's bytes form a sub-plane at byte
 *            16 * (group g's byte offset in a row); a row's group bytes split
 *            into octets of b_g bytes (8 indices each), and octet o of row t
 *            sits in run (m/8)*(t % 4) + o of 4*b_g bytes, at place t / 4
 *            (byte q of it at run start + (t / 4)*b_g + q).  Other V formats
 *            use the K layout.
 */

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* tq_last_error(void);

/*
 * Fill out_f16[0 .. 2^bits) with the fp16 Lloyd-Max levels of a unit
 * Gaussian (ascending, exactly symmetric), computed on the host in extended
 * precision and rounded to nearest even ([S "Architecture notes"]: Lloyd-Max
 * codebooks are computed once on the CPU).  bits in 1..4.
 * Errors: VALUE for bits out of range or a NULL pointer.
 */
tq_status tq_lloyd_max_codebook(int32_t bits, uint16_t* out_f16 /* host */);

/* Check a format descriptor (VALUE on any malformed field). */
tq_status tq_format_check(const tq_format* fmt /* host */);

/*
 * Byte math of a format ([D "Serving Route Design"]).  block_size must be 16.
 *   row_index_bytes = sum over groups of m * bits / 8 (+ head_dim / 8 with qjl)
 *   tile_bytes      = roundup16(16 * row_index_bytes + 16 * num_groups * 2
 *                               (* 2 with qjl: residual norms))
 */
tq_status tq_tile_bytes(const tq_format* fmt, int32_t block_size, int32_t* row_index_bytes /* host out */,
                        int32_t* tile_bytes /* host out */);

/*
 * Quantise-on-write ([D "Serving Route Design"]: the serving route writes
 * packed rows into persistent pages).  For token i and kv head h the row
 * k[i][h][0..head_dim) (resp. v) is encoded with kfmt (resp. vfmt) and stored
 * at block slot_mapping[i] / 16, offset slot_mapping[i] % 16 of head h.
 *
 *   k, v          device, [num_tokens][num_kv_heads][head_dim] contiguous,
 *                 in_dtype TQ_BF16 or TQ_F32.  Either may be NULL (then its
 *                 pages and format are ignored), not both.
 *   slot_mapping  device int64 [num_tokens]; slots must be distinct within a
 *                 call (documented precondition, not checked).
 *   k_pages/v_pages  device pools [num_blocks][num_kv_heads][tile_bytes].
 *   dev_err       device int32[2] or NULL: a slot outside
 *                 [0, num_blocks*16) records (TQ_ERR_INDEX, token index) and
 *                 that token's rows are not written.
 * A K format with the QJL stage adds a second kernel on the same stream
 * that computes each written row's residual, signs and residual norm.
 * Status: VALUE (shapes, dtype, formats, NULLs, qjl set on the V format,
 * qjl_proj NULL or not 16-byte aligned), UNSUPPORTED_FORMAT (block_size !=
 * 16), DEVICE (launch failure), else OK.
 */
tq_status tq_write_kv(const void* k, const void* v, tq_dtype in_dtype, int64_t num_tokens,
                      int32_t num_kv_heads, const int64_t* slot_mapping, uint8_t* k_pages,
                      uint8_t* v_pages, int64_t num_blocks, int32_t block_size, const tq_format* kfmt,
                      const tq_format* vfmt, int32_t* dev_err, tq_stream_t stream);

/*
 * Device self-test of the write path's arithmetic (diagnostics; the bit
 * exact encoding above rests on it): for i < n, out_sqrt[i] = sqrt(a[i]),
 * out_div[i] = a[i] / b[i], out_mul[i] = a[i] * b[i] (each IEEE binary64,
 * correctly rounded) and out_f16[i] = the binary16 bits of a[i] rounded to
 * nearest, ties to even, directly from binary64 -- computed by a kernel
 * built like the write kernel (no fused multiply-add).  A caller compares
 * them with any IEEE host.  All pointers device; n in [0, 2^31); VALUE on a
 * bad argument.
 */
tq_status tq_selftest_fp64(const double* a, const double* b, int64_t n, double* out_sqrt, double* out_div,
                           double* out_mul, uint16_t* out_f16, tq_stream_t stream);

/*
 * Workspace of tq_decode_paged: num_seqs * num_q_heads * num_splits *
 * (head_dim + 1) * 4 bytes when num_splits > 1, else 0.  It depends on the
 * runtime shape only, never on context length ([D "Serving Route Design"]:
 * the workspace is bounded by the runtime shape).
 */
tq_status tq_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                    int32_t num_splits, uint64_t* bytes /* host out */);

/*
 * Paged decode attention over packed pages ([D "Serving Route Design"]: block
 * tables map logical to physical blocks, K rows are read inside the score
 * computation and V rows are dequantised inside the accumulation; no dense
 * K/V history is ever built).
 *
 *   q            device [num_seqs][num_q_heads][head_dim], q_dtype BF16/F32.
 *   q head h attends with kv head h / (num_q_heads / num_kv_heads).
 *   block_tables device int32 [num_seqs][max_blocks_per_seq]; entry b of
 *                sequence s is the physical block of its tokens 16b..16b+15.
 *                Entries at or beyond ceil(context_lens[s] / 16) are not read.
 *   context_lens device int32 [num_seqs]: cached tokens per sequence (the
 *                current token included: write it first).
 *   scale        softmax scale applied to q.k.
 *   num_splits   P >= 1: the most pieces one (sequence, kv head) may be cut
 *                into.  The work (sequence, kv-head group, logical block) is
 *                split evenly over one persistent workgroup per CU, each
 *                segment charged a fixed number of extra blocks for the cost
 *                of starting a piece; a range of at least
 *                ceil(max_blocks_per_seq / (P - 1)) positions each keeps
 *                every segment within P pieces (P == 1: ranges end at segment
 *                boundaries, nothing is split).  A cut segment leaves one
 *                partial (o_p, lse_p) per piece in the workspace and the
 *                partials are merged by log-sum-exp inside this call.
 *                workspace must hold tq_decode_workspace_bytes() bytes
 *                (device, may be NULL when P == 1); its contents on entry
 *                do not matter (every slot the merge reads is written first:
 *                an uncut row's slot 0 holds a marker, the slots past a cut
 *                segment's last piece hold -inf).
 *   out          device [num_seqs][num_q_heads][head_dim], out_dtype BF16/F32.
 *   lse          device float [num_seqs][num_q_heads] or NULL: natural-log
 *                sum of exp(scale * q.k) over the context.
 *   dev_err      device int32[2] or NULL: a block-table entry outside
 *                [0, num_blocks) records (TQ_ERR_INDEX, s*max_blocks_per_seq+b)
 *                and the block is skipped; a context length outside
 *                [0, 16*max_blocks_per_seq] records (TQ_ERR_INDEX, -1 - s) and
 *                is clamped.
 * A sequence with context length 0 gets out = 0 and lse = -inf.
 * Served formats (else UNSUPPORTED_FORMAT): head_dim 64 or 128; K one group
 * of 4 or 2 bits, or two groups of 4 + 3 bits (3.5-bit recipe) or 3 + 2 bits
 * (2.5-bit recipe; [S "What it does"], [D "Recipe Strategy"]); V the same
 * four (the formats independent, [D "System Invariants"]);
 * num_q_heads / num_kv_heads in 1..TQ_MAX_COLUMNS (1..64 with the QJL
 * stage; see below); block_size 16.  Each page pool must be smaller than 4 GiB and
 * num_blocks below 2^31 (else VALUE).
 * Results are reproducible up to the order of floating-point accumulation:
 * blocks are shared dynamically among the waves serving a kv head.
 * K formats with the QJL stage (qjl = 1) add the sign sketch's term to
 * every score.  With K groups of 4, 2, 4+3 or 3+2 bits and a one-group V
 * format the same kernel serves them (the projected query on the matrix
 * cores, up to 64 (query, q head) pairs per kv head); other QJL layouts (K
 * bits 2-4 in any grouping) run a separate kernel with one workgroup per
 * (sequence, kv head, split p), split p taking logical blocks [p*c,
 * (p+1)*c), c = ceil(ceil(context_lens[s] / 16) / P), every split writing
 * its partial (lse -inf when empty) before the same merge; that kernel takes
 * one query and at most 8 q heads per kv head, and 16-byte aligned page
 * pools.  qjl_proj must be 16-byte aligned (else VALUE).  Two-group V with
 * a QJL K format is UNSUPPORTED_FORMAT.
 */
tq_status tq_decode_paged(const void* q, tq_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_kv_heads, const uint8_t* k_pages, const uint8_t* v_pages,
                          int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          const tq_format* kfmt, const tq_format* vfmt, float scale,
                          int32_t num_splits, void* workspace, uint64_t workspace_bytes, void* out,
                          tq_dtype out_dtype, float* lse, int32_t* dev_err, tq_stream_t stream);

/*
 * Multi-query paged decode: num_queries new tokens per sequence attend the
 * packed pages causally in one call (chunked prefill / several draft tokens
 * per step; the "next" workload after single-query decode).  Reading: the
 * sequence's last num_queries cached tokens are the queries' own (write
 * them first, as for tq_decode_paged), so query i (0-based) attends tokens
 * [0, context_lens[s] - (num_queries - 1 - i)); a query left with no token
 * gets out = 0 and lse = -inf.  The (query, q head) pairs of a kv head share
 * the matrix-core columns of the kv head's workgroup, 8 per group of
 * waves, so every page is read from memory once for all queries (the waves
 * of the column groups read each tile at about the same time).
 *   q, out       device [num_seqs][num_queries][num_q_heads][head_dim].
 *   lse          device float [num_seqs][num_queries][num_q_heads] or NULL.
 *   workspace    tq_decode_workspace_bytes(num_seqs * num_queries, ...).
 * Every other argument, error and format is as for tq_decode_paged, which
 * is this call with num_queries = 1.  Served: num_queries * (num_q_heads /
 * num_kv_heads) <= TQ_MAX_COLUMNS (64 for a K format with the QJL stage;
 * one query and 8 q heads for the QJL layouts of the separate kernel, see
 * tq_decode_paged), else UNSUPPORTED_FORMAT.
 */
tq_status tq_decode_paged_multi(const void* q, tq_dtype q_dtype, int32_t num_seqs, int32_t num_queries,
                                int32_t num_q_heads, int32_t num_kv_heads, const uint8_t* k_pages,
                                const uint8_t* v_pages, int64_t num_blocks, int32_t block_size,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, const tq_format* kfmt, const tq_format* vfmt,
                                float scale, int32_t num_splits, void* workspace, uint64_t workspace_bytes,
                                void* out, tq_dtype out_dtype, float* lse, int32_t* dev_err, tq_stream_t stream);

/*
 * tq_decode_paged without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It allocates nothing: the split
 * partials go to a device array of TQ_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends (its address
 * is looked up on the first call on each device).  The call runs on the
 * current device; `stream` must belong to it.  Every argument, format and
 * error is as for tq_decode_paged, plus VALUE when the split workspace
 * (tq_decode_workspace_bytes) would exceed TQ_NOALLOC_SCRATCH_BYTES.  All
 * calls on one GPU share the one array, which keeps the last call's
 * contents: calls that overlap on one GPU (concurrent streams, threads)
 * race and give undefined results; calls on one stream are ordered.
 */
#define TQ_NOALLOC_SCRATCH_BYTES (16ull << 20)
tq_status tq_decode_paged_noalloc(const void* q, tq_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, const uint8_t* k_pages, const uint8_t* v_pages,
                                  int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  const tq_format* kfmt, const tq_format* vfmt, float scale,
                                  int32_t num_splits, void* out, tq_dtype out_dtype, float* lse,
                                  int32_t* dev_err, tq_stream_t stream);

/*
 * Log-sum-exp merge of split partials (flash-decoding):
 *   lse = M + ln sum_p exp(lse_p - M),  out = sum_p exp(lse_p - lse) * o_p
 *   part_out  device float [num_seqs][num_heads][num_splits][head_dim]
 *             (normalised partial outputs, original domain)
 *   part_lse  device float [num_seqs][num_heads][num_splits]; -inf marks an
 *             empty partial, whose part_out row is not read.  All partials
 *             empty: out = 0, lse = -inf.
 *   out       device [num_seqs][num_heads][head_dim], BF16 or F32.
 *   lse       device float [num_seqs][num_heads] or NULL.
 */
tq_status tq_split_merge(const float* part_out, const float* part_lse, int32_t num_seqs,
                         int32_t num_heads, int32_t num_splits, int32_t head_dim, void* out,
                         tq_dtype out_dtype, float* lse, tq_stream_t stream);

/*
 * Exact attention over a dense window of cached tokens, optionally merged
 * with the packed history's result ([D "Format Strategy"]: a recent dense
 * window and boundary-token preservation are among the first serving
 * policies; [D "Data Ownership"]: the compressed cache owns its recent
 * windows next to the compressed blocks).  Reading: the window holds a
 * sequence's boundary (first) tokens and its most recent tokens unquantised;
 * they are attended exactly in the original domain and combined with the
 * packed history by the split merge's log-sum-exp identity.  The tokens of
 * a window may sit in any order (attention over a set of tokens does not
 * depend on their order) and must not also be in the pages.
 *
 *   q          device [num_seqs][num_q_heads][head_dim], q_dtype BF16/F32
 *              (the same q as tq_decode_paged).
 *   k, v       device [num_seqs][capacity][num_kv_heads][head_dim], kv_dtype
 *              BF16/F32, 16-byte aligned; token t of sequence s at row
 *              (s * capacity + t); may be NULL when capacity == 0.
 *   lens       device int32 [num_seqs]: tokens held for each sequence, at
 *              rows 0 .. lens[s]-1; a length outside [0, capacity] records
 *              (TQ_ERR_INDEX, -1 - s) in dev_err and is clamped.
 *   scale      softmax scale applied to q.k (finite, > 0).
 *   hist_out   device float [num_seqs][num_q_heads][head_dim] and
 *   hist_lse   device float [num_seqs][num_q_heads], both or neither: the
 *              history's normalised output and natural-log lse (for example
 *              tq_decode_paged with out_dtype F32 and lse).  A -inf hist_lse
 *              marks an empty history, whose hist_out row is not read.
 *              NULL: the result is the window's attention alone.
 *   out        device [num_seqs][num_q_heads][head_dim], out_dtype BF16/F32,
 *              8-byte aligned; may be hist_out itself (F32), and lse may be
 *              hist_lse: every row is read before it is written.
 *   lse        device float [num_seqs][num_q_heads] or NULL.
 * History and window both empty: out = 0, lse = -inf.
 * Served shapes (else UNSUPPORTED_FORMAT): head_dim 64 or 128, num_q_heads /
 * num_kv_heads in 1..16.  One workgroup per (sequence, kv head); the window
 * is walked in chunks of 256 tokens, so capacity has no upper limit other
 * than memory.
 */
tq_status tq_decode_dense(const void* q, tq_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, const void* k, const void* v,
                          tq_dtype kv_dtype, int32_t capacity, const int32_t* lens, float scale,
                          const float* hist_out, const float* hist_lse, void* out,
                          tq_dtype out_dtype, float* lse, int32_t* dev_err, tq_stream_t stream);

/*
 * The packed history and a dense bf16 window attended in ONE call: the
 * result of tq_decode_paged over the pages followed by tq_decode_dense over
 * the window with that history (same readings: [D "Format Strategy"] and
 * [D "Data Ownership"], window tokens are not also in the pages).  The
 * persistent workgroups of the paged decode take the (sequence, kv head)
 * window items after their pages; each item's normalised output and lse go
 * to one more partial slot of its rows, and the split merge combines every
 * row's slots by the log-sum-exp identity.
 *   q ... vfmt   as for tq_decode_paged (one query per sequence).
 *   win_k, win_v device [num_seqs][win_capacity][num_kv_heads][head_dim],
 *                win_dtype BF16 (else UNSUPPORTED_FORMAT: tq_decode_dense
 *                takes f32 windows), 16-byte aligned; may be NULL when
 *                win_capacity == 0.
 *   win_lens     device int32 [num_seqs]: window tokens of sequence s at rows
 *                0 .. win_lens[s]-1; outside [0, win_capacity] records
 *                (TQ_ERR_INDEX, -1 - s) in dev_err and is clamped.
 *   workspace    tq_decode_workspace_bytes(num_seqs, num_q_heads, head_dim,
 *                num_splits + 1) bytes (needed even for num_splits == 1).
 *   out, lse     as for tq_decode_paged; history and window both empty:
 *                out = 0, lse = -inf.
 * Served: num_q_heads / num_kv_heads <= 16 and the formats of the main
 * decode kernel (not the QJL layouts of the separate kernel), else
 * UNSUPPORTED_FORMAT.
 */
tq_status tq_decode_paged_window(const void* q, tq_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, const uint8_t* k_pages, const uint8_t* v_pages,
                                 int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens, const tq_format* kfmt,
                                 const tq_format* vfmt, const void* win_k, const void* win_v, tq_dtype win_dtype,
                                 int32_t win_capacity, const int32_t* win_lens, float scale, int32_t num_splits,
                                 void* workspace, uint64_t workspace_bytes, void* out, tq_dtype out_dtype,
                                 float* lse, int32_t* dev_err, tq_stream_t stream);

/*
 * Phase timestamps of the paged decode kernel, for performance analysis
 * only.  In a library built with TQ_PHASE_TRACE defined, every later
 * tq_decode_paged / tq_decode_paged_multi call served by the main decode
 * kernel (every format but the QJL layouts of the separate kernel) has thread
 * 0 of each persistent workgroup w write 16 uint64 values to
 * buf[16 w .. 16 w + 15]: the 100 MHz real-time counter at kernel entry
 * (0), when the work split is known (1), per piece i < 3 at its start
 * (2 + 4i), at the start (3 + 4i) and end (4 + 4i) of its block loop and at
 * the end of its epilogue (5 + 4i), at exit (14), and the number of pieces
 * (15).  buf: device, at least 16 * (number of CUs) values, or NULL to stop.
 * Status: OK, or UNSUPPORTED_FORMAT in a library built without the option
 * (the normal build; the pointer is then ignored).
 */
tq_status tq_debug_phase_trace(uint64_t* buf /* device, nullable */);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
