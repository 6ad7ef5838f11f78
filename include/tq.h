/*
 * tq.h -- C ABI of the TurboQuant hot path on MI355X (gfx950).
 *
 * TurboQuant (Zandieh et al., "TurboQuant: Online Vector Quantization with
 * Near-optimal Distortion Rate", ICLR 2026) compresses vectors by a random
 * rotation followed by per-coordinate Lloyd-Max quantization; keys also get a
 * 1-bit QJL sign projection of the residual so that inner products with a
 * full-precision query are estimated without bias.
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device memory owned by the caller.  The library
 *     never allocates, frees or keeps a pointer after a call returns, never
 *     synchronises the device, and enqueues all work on the given stream
 *     (a hipStream_t passed as void*; NULL is the null stream).
 *   - Host pointers are read during the call only.
 *   - Every argument is validated on the host before anything is launched.
 *     A bad argument returns TQ_ERR_INVALID_ARG, a shape the kernels do not
 *     implement returns TQ_ERR_UNSUPPORTED, and in both cases nothing is
 *     launched.  A failed launch returns TQ_ERR_HIP.  tq_last_error() gives a
 *     thread-local message for the last non-OK status.
 *   - Calls may be made from any thread.  The library keeps no mutable state
 *     between calls, apart from tq_scores_noalloc's per-device scratch array
 *     (and its address, resolved once per device).
 *
 * Packed records (the layout the pages' storage accounting implies: b bits
 * per coordinate of codes, one sign bit per projection row, float16 norms):
 *   bit-planes of 32-bit little-endian words, coordinate j of plane p at bit
 *   (j mod 32) of word (j div 32) of that plane; the P planes of a record are
 *   interleaved word by word, word w of plane p being u32 number w * P + p of
 *   the record (the P words covering one group of 32 coordinates are adjacent):
 *     key   (prod, b bits)  planes 0 .. b-2 = bit p of the (b-1)-bit index,
 *                           plane b-1      = QJL bits, 1 <=> (S r)_i >= 0;
 *                           scalars = { float16 n = ||x||, float16 gamma = ||r|| }
 *     value (mse,  b bits)  planes 0 .. b-1 = bit p of the b-bit index;
 *                           scalars = { float16 n }
 *     MSE-only key (b bits) the value record in the key cache's per-record
 *                           layout (tq_encode_mse_keys)
 *   A key cache holds the plane words of all records in one array, u32
 *   [records][d_rot/32][P], and the scalars in another, f16
 *   [records][scalars]; record r of segment s is s * seg_stride + t.
 *   A value cache stores the same bits transposed in blocks of 32 records
 *   (values are read along tokens): u32 [ceil(records/32)][d_rot][P], word
 *   (B, j, p) holding in bit i the bit p of the index of record 32 B + i at
 *   coordinate j; scalars f16 [records][1].  seg_stride of a value cache must
 *   be a multiple of 32 so that segments start on a block.
 *   At d = 128, b = 3 a key record is 48 + 4 bytes and a value 48 + 2 bytes.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = 1,
  TQ_ERR_UNSUPPORTED = 2,
  TQ_ERR_HIP = 3
} tq_status;

/* Rotations: a dense orthogonal matrix; the sign-flipped Hadamard transform
 * (one round); or two rounds of it with independent signs. */
typedef enum { TQ_ROT_DENSE = 0, TQ_ROT_HADAMARD = 1, TQ_ROT_HADAMARD2 = 2 } tq_rot;
/* Values of the int dtype and layout arguments (passed as int so that any
 * value a caller passes is defined and rejected when it names none of these). */
typedef enum { TQ_F32 = 0, TQ_F16 = 1 } tq_dtype;
/* Record layout of an MSE encode (tq_encode_eden). */
typedef enum { TQ_LAYOUT_BLOCKS = 0, TQ_LAYOUT_RECORDS = 1 } tq_layout;

/* Parameters of one quantizer (one for keys, one for values).
 *   d       input dimension
 *   d_rot   rotated dimension: == d for the dense rotation; a power of two
 *           >= d for the Hadamard rotation (inputs are zero-padded at the end)
 *   m       QJL projection rows (prod only, else ignored): d_rot, or d_rot / 2
 *           (the first page's proj_dim = head_dim / 2) at d_rot = 128 (encode,
 *           tq_scores, tq_attend) and d_rot = 2048 (encode, tq_scores_topk)
 *   bits    total bit budget b: prod uses b-1 index bits plus 1 QJL bit
 *           (2 <= b <= 4), mse uses b index bits (1 <= b <= 4)
 *   rot     TQ_ROT_DENSE, TQ_ROT_HADAMARD (y = H D pad(u) / sqrt(d_rot)) or
 *           TQ_ROT_HADAMARD2 (two rounds: y = (H D2 / sqrt(d_rot)) (H D1 /
 *           sqrt(d_rot)) pad(u), round 1 first, D_r = diag(eps[r]); the
 *           explainer page's randomised Hadamard transform applied twice).
 *           Two rounds run natively at d_rot = 2048; at d_rot = 128 pass the
 *           matrix of tq_hadamard_matrix as a dense pi instead.
 *   pi      device f32 [d_rot][d] row-major, y = pi * u   (dense; else NULL)
 *   eps     device f32 [rounds][d_rot] of +1/-1          (hadamard; else NULL)
 *   s       device f32 [m][d_rot] row-major, the Gaussian QJL matrix (prod; NULL for mse)
 *   centroids   HOST f32 [2^bq] ascending, bq = index bits, unit-sphere units
 *   boundaries  HOST f32 [2^bq - 1], centroids[i] < boundaries[i] < centroids[i+1]
 *   n_sets, set_div   rotation sets (0 or 1: one set).  pi, eps and s may
 *           hold n_sets consecutive sets ([n_sets][d_rot][d], [n_sets][d_rot],
 *           [n_sets][m][d_rot]); segment seg of tq_scores and tq_attend uses
 *           set (seg / set_div) % n_sets: per layer, set_div = KV heads per
 *           layer and n_sets = layers; per (layer, head), set_div = 1 and
 *           n_sets = segments; per head shared by all layers, set_div = 1 and
 *           n_sets = heads (segments ordered layer-major).  The encoders use
 *           the set the pointers name: encode each set's vectors with a
 *           tq_params whose pointers point at that set.  tq_scores_topk takes
 *           one set.  (The first page uses one key and one value rotation for
 *           all layers; independent per-layer or per-head rotations are the
 *           variant its storage/variance discussion leaves open.)
 * The score and attend kernels also require the codebook to be odd-symmetric
 * (centroids[2^bq-1-i] == -centroids[i], boundaries likewise), which every
 * Lloyd-Max codebook of this density is (TQ_ERR_UNSUPPORTED otherwise). */
typedef struct {
  int d;
  int d_rot;
  int m;
  int bits;
  int rot;
  const float* pi;
  const float* eps;
  const float* s;
  const float* centroids;
  const float* boundaries;
  int n_sets;
  int set_div;
} tq_params;

/* A packed cache, device memory owned by the caller (layout above).
 * seg_stride is the number of records between consecutive segments; it is
 * used by tq_scores / tq_attend and ignored by the encoders.
 * records is the capacity: the number of records planes and scalars hold (a
 * value cache's planes hold ceil(records / 32) blocks).  The encoders write
 * no record at or past it (a slot outside [0, records) is skipped on the
 * device), and the decode calls return TQ_ERR_INVALID_ARG when the records
 * they would read do not fit in it. */
typedef struct {
  void* planes;
  void* scalars;
  int64_t seg_stride;
  int64_t records;
} tq_cache;

const char* tq_status_string(int s);
const char* tq_last_error(void);

/* Lloyd-Max codebook for one coordinate of a uniformly rotated unit vector
 * in R^d, whose density is Gamma(d/2)/(sqrt(pi) Gamma((d-1)/2)) (1-x^2)^((d-3)/2)
 * on [-1, 1] (blog notes on the TurboQuant paper, Lemma 1 and eq. (4); the
 * explainer page, section 5: boundaries at midpoints, centroids at the
 * conditional means).  d == 0 gives the N(0,1) codebook (the limit of
 * sqrt(d) * c as d grows).  Host only, float64, deterministic, exactly
 * odd-symmetric.  d in {0} U [2, 65536], 1 <= bits <= 4.
 * centroids: host double[2^bits] (ascending), boundaries: host double[2^bits-1]. */
tq_status tq_build_codebook(int d, int bits, double* centroids, double* boundaries);

/* The R-round sign-flipped Hadamard transform as an explicit matrix:
 *   out[i][j] = ((H D_R / sqrt(d_rot)) ... (H D_1 / sqrt(d_rot)) e_j)_i,
 * i < d_rot, j < d (the zero padding of inputs shorter than d_rot folded in),
 * D_r = diag(eps[r]), H the Sylvester Hadamard matrix.  Passed as a dense
 * rotation (rot = TQ_ROT_DENSE, pi = out, d_rot = d) it gives the encoders,
 * scores and attention at d = 128 the multi-round transform.  The unscaled
 * transform is exact in float32; the scale d_rot^(-R/2) is applied once, so
 * the two-round matrix (entries integer / d_rot) is exact.
 * eps     device f32 [rounds][d_rot] of +1/-1
 * out     device f32 [d_rot][d] (written)
 * Supported: d_rot a power of two in [2, 2048], 1 <= d <= d_rot, 1 <= rounds <= 2.
 * One launch on the stream. */
tq_status tq_hadamard_matrix(const float* eps, int rounds, int d, int d_rot, float* out, void* stream);

/* Number of 32-bit plane words and float16 scalars in one record.  For a key
 * quantizer without a QJL matrix (s == NULL) tq_key_layout describes MSE-only
 * key records: b planes and one scalar.  With m = d_rot / 2 QJL rows the sign
 * plane has m / 32 words (see tq_key_record_words). */
tq_status tq_key_layout(const tq_params* p, int* planes, int* words_per_plane, int* scalars);
tq_status tq_value_layout(const tq_params* p, int* planes, int* words_per_plane, int* scalars);

/* 32-bit words of one key record, 0 for invalid parameters.  A prod record
 * holds, for each group of 32 coordinates w = 0 .. d_rot/32 - 1, the b-1 index
 * words of the group and then sign word w if w < m/32 (the first page's
 * proj_dim = head_dim / 2 default gives m/32 = 2 at d = 128: 40 bytes of
 * words at b = 3 instead of 48); with m = d_rot this is the interleaved layout
 * above.  MSE-only key records hold b words per group. */
size_t tq_key_record_words(const tq_params* p);

/* Bytes of one key record (plane words plus float16 scalars) and of one value
 * record (its share of the block words plus its float16 norm), 0 for invalid
 * parameters: the storage accounting of the first page's memory formula
 * (52 and 50 bytes at d = 128, b = 3; 5.02x smaller than float16 K and V). */
size_t tq_key_record_bytes(const tq_params* p);
size_t tq_val_record_bytes(const tq_params* p);

/* TurboQuant-prod encode of n vectors (keys) into a packed cache.
 * Blog notes on the paper, the Q_prod definition; explainer page section 8:
 *   n_x = ||x||, u = x/n_x (0 if n_x = 0), y = rot(u),
 *   idx = #{boundaries <= y} at b-1 bits, r = y - c[idx], gamma = ||r||,
 *   z = [S r >= 0]; stores float16 n_x and gamma (round to nearest even).
 * x      device [n][ld_x] of dtype (f32 or f16), rows are vectors, ld_x >= d
 * slot   device int64 [n] record index for each vector, or NULL for 0..n-1
 * out    cache with planes/scalars of p's key layout and out.records >= 1;
 *        a vector whose record index lies outside [0, out.records) is not
 *        written
 * Supported: d_rot = 128 (dense or Hadamard) and Hadamard d_rot = 2048. */
tq_status tq_encode_prod(const tq_params* p, const void* x, int dtype, int64_t n,
                         int64_t ld_x, tq_cache out, const int64_t* slot, void* stream);

/* Workspace bytes tq_encode_prod_ws needs for n vectors: 0 at d_rot = 128;
 * at d_rot = 2048 (Hadamard) the QJL matrix split into fp16 hi/lo (16 MiB)
 * plus a chunk of up to 32768 residual rows (fp16 hi/lo, 128 KiB each). */
size_t tq_encode_workspace(const tq_params* p, int64_t n);

/* tq_encode_prod with a caller-owned workspace (device, 256-B aligned, no
 * initial contents, at least tq_encode_workspace(p, n) bytes, one call in
 * flight per workspace).  Needed for the retrieval configuration, d_rot = 2048
 * with the sign-flipped Hadamard rotation (d <= 2048, a multiple of 8,
 * zero-padded): pass 1 runs the 2048-point Walsh-Hadamard transform in
 * registers (one wave per vector) and quantises; pass 2 forms the QJL
 * projection S r of each chunk of residuals on the matrix cores.  Records use
 * the key layout of tq_key_layout (W = 64 words per plane); with m = 1024 QJL
 * rows, the tq_key_record_words layout (sign words in groups 0..31 only). */
tq_status tq_encode_prod_ws(const tq_params* p, const void* x, int dtype, int64_t n,
                            int64_t ld_x, tq_cache out, const int64_t* slot, void* ws,
                            size_t ws_bytes, void* stream);

/* TurboQuant-MSE encode (values): as above without the QJL stage, b index
 * bits, written in the blocked value layout.  A group of 32 vectors that fills
 * one aligned block (slot NULL, or slots base + 0..31 with base a multiple of
 * 32) is written with whole-word stores; any other record updates only its
 * own bit of each word, so partial blocks keep their other records.  In calls
 * of up to 4096 vectors a block that exactly one group of 32 consecutive
 * vectors of the call writes is updated by reading, changing and storing
 * whole words; other blocks take per-bit atomic clear/set.  Two calls in
 * flight at once (different streams) must therefore not write records of the
 * same 32-record block; calls on one stream are ordered and always safe.
 * At d_rot = 2048 with the sign-flipped Hadamard rotation (d a multiple of 8,
 * d <= 2048) the records instead use the per-record key layout of
 * tq_key_layout with b planes and one fp16 scalar ||x||_2 per record (no
 * workspace, one launch, one wave per vector); these are the MSE-only
 * retrieval records read by tq_scores_topk. */
tq_status tq_encode_mse(const tq_params* p, const void* x, int dtype, int64_t n,
                        int64_t ld_x, tq_cache out, const int64_t* slot, void* stream);

/* TurboQuant-MSE encode of keys (blog notes on the paper, Q_mse: the
 * quantizer without the QJL stage whose bias that stage removes, explainer
 * page section 8) into the per-record key layout: b index planes (1 <= b <= 4)
 * and one float16 n per record, written whole per record (any slot order, no
 * atomics).  p->s is ignored (NULL by convention: tq_key_layout, tq_scores and
 * tq_attend read a key quantizer without s as MSE-only).  Arguments as for
 * tq_encode_prod.  Supported: d = d_rot = 128 (dense or Hadamard), and the
 * Hadamard rotation at d_rot = 2048, where the records are those of
 * tq_encode_mse. */
tq_status tq_encode_mse_keys(const tq_params* p, const void* x, int dtype, int64_t n,
                             int64_t ld_x, tq_cache out, const int64_t* slot, void* stream);

/* MSE encode with EDEN's unbiased per-vector scale (the prior-work map of the
 * explainer page, section 0.9: EDEN keeps S = ||x||^2 / <R x, Q(R x)>, which
 * makes the reconstruction unbiased; at one bit it is DRIVE's unbiased scale
 * ||x||^2 / ||R x||_1).  The codes are those of tq_encode_mse; the record's
 * fp16 scalar holds, in place of n = ||x||,
 *   S = n / <y, c[idx]>      (y = rot(x / n), c the unit-sphere centroids),
 * so the dequantized vector S rot^T(c[idx]) has <x, x^> = ||x||^2 exactly and
 * E[x^] = x over the rotation, and the score and attention calls, which read
 * the scalar as they read n, return unbiased estimates.  S = 0 for x = 0.
 * layout  TQ_LAYOUT_BLOCKS: values in the token-blocked layout (as
 *         tq_encode_mse); TQ_LAYOUT_RECORDS: MSE-only keys in the per-record
 *         key layout (as tq_encode_mse_keys)
 * Other arguments as for tq_encode_mse.  Supported: d = d_rot = 128, and the
 * Hadamard rotation at d_rot = 2048, whose MSE records are always per record
 * (the retrieval records of tq_scores_topk with kp->s == NULL; layout is
 * ignored there). */
tq_status tq_encode_eden(const tq_params* p, const void* x, int dtype, int64_t n, int64_t ld_x,
                         int layout, tq_cache out, const int64_t* slot, void* stream);

/* Workspace bytes tq_scores needs for segs segments of group query heads. */
size_t tq_scores_workspace(const tq_params* kp, int segs, int group);

/* Asymmetric scores of query heads against packed prod keys (explainer
 * page section 8; blog notes, the prod estimator read with ||r||_2):
 *   s[h][t] = n_t ( <rot(q_h), c[idx_t]> + gamma_t sqrt(pi/2)/m <S rot(q_h), 2 z_t - 1> )
 * for query head h of segment h / group and token t < len[h / group].
 * With kp->s == NULL the keys are MSE-only records (tq_encode_mse_keys, b
 * index bits, b = 1..4) and the estimate is the MSE inner product
 *   s[h][t] = n_t <rot(q_h), c[idx_t]>    (biased; no QJL term).
 * q       device f32 [segs*group][d]
 * keys    packed prod cache, segment s at records s*seg_stride + t
 * len     device int32 [segs] valid tokens per segment (<= T), or NULL for T
 * scores  device f32 [segs*group][T]; entries with t >= len are not written
 * ws      device workspace of at least tq_scores_workspace() bytes, 256-B
 *         aligned, no initial contents required; it receives each segment's
 *         query pack (rotated and projected query heads quantised to the
 *         matrix-core operand) and four hand-over words per segment, so one
 *         call in flight per workspace.
 * One launch on the stream when the pass fits in one dispatch of the device's
 * 8-wave workgroups (one per 2048 tokens of each segment); a longer pass runs
 * as two launches on the stream, the query packs and then the pass, and leaves
 * the hand-over words untouched.  In the one launch, per segment, the first
 * workgroup builds the query pack while the others already stream their first
 * keys; they take the pack
 * when its builder publishes a per-call ticket in the workspace.  The pack and
 * the ticket words are written and read with device-coherent (sc1) accesses
 * and relaxed device-scope atomics, so no cache flush is needed.  A workgroup
 * that has waited 200 us without the pack (its producer not yet resident)
 * claims the pack and builds it itself; exactly one workgroup per segment and
 * call writes the pack.  Each call leaves the ticket words cleared, so a
 * captured launch can be replayed. */
tq_status tq_scores(const tq_params* kp, const float* q, int segs, int group, tq_cache keys,
                    const int32_t* len, int64_t T, float* scores, void* ws, size_t ws_bytes,
                    void* stream);

/* tq_scores for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same call and
 * results without the workspace arguments.  Its workspace is a device array
 * inside the library, tq_scores_noalloc_capacity() bytes (16 MiB) on each GPU,
 * held until the process ends and resolved with hipGetSymbolAddress on a
 * device's first call; nothing is allocated or freed.  Every call on a GPU
 * uses that GPU's one array, so calls that overlap on one GPU (other streams,
 * other threads) race: serialise them.  The array keeps the last call's
 * contents; the hand-over words need no clearing (the per-call ticket).
 * Returns TQ_ERR_UNSUPPORTED when segs and group need a larger workspace than
 * the array (tq_scores_workspace > capacity), before any launch. */
tq_status tq_scores_noalloc(const tq_params* kp, const float* q, int segs, int group, tq_cache keys,
                            const int32_t* len, int64_t T, float* scores, void* stream);
size_t tq_scores_noalloc_capacity(void);

/* The two halves of tq_scores, for callers that time them apart or score the
 * same queries against several caches: tq_scores_prepare writes the query
 * pack of every segment into ws (arguments as for tq_scores);
 * tq_scores_prepared streams the keys against the pack ws holds (from the last
 * tq_scores_prepare with the same kp, segs and group on this workspace). */
tq_status tq_scores_prepare(const tq_params* kp, const float* q, int segs, int group, void* ws,
                            size_t ws_bytes, void* stream);
tq_status tq_scores_prepared(const tq_params* kp, int segs, int group, tq_cache keys, const int32_t* len,
                             int64_t T, float* scores, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes tq_attend needs. */
size_t tq_attend_workspace(const tq_params* kp, const tq_params* vp, int segs, int group, int64_t T);

/* Softmax attention of query heads over a packed cache (first page, usage
 * pattern 1: scores from the compressed keys, softmax, weighted sum of the
 * MSE-dequantized values):
 *   p = softmax_t(scale * s[h][t]) over t < len,  o[h] = sum_t p_t n_v,t rot_v^T(c_v[idx_v,t])
 * computed as one rot_v^T per head after accumulating in the rotated domain.
 * out     device f32 [segs*group][d]; a segment with len 0 gives zeros
 * vals    packed mse value cache (block layout), vals.seg_stride a multiple of
 *         32 and, like keys.seg_stride, >= T; its scalars must cover
 *         segs * seg_stride records
 * Other arguments as for tq_scores (ws: tq_attend_workspace() bytes).  Three
 * launches: the query pack, the streaming pass (one log-sum-exp partial per
 * workgroup) and the per-segment merge with the inverse value rotation.
 * Supported: d = 128, group <= 16, value bits 1..4.  With kp->s == NULL the
 * keys are MSE-only records (tq_encode_mse_keys) scored as in tq_scores;
 * then key and value bits are 2..4, and 4-bit keys take group <= 8 or an even
 * group <= 16 (run as two halves of group / 2 heads that each read the
 * segment's keys and values, so such a call reads the cache twice).  Prod
 * keys with m = d_rot / 2 take value bits 2..4. */
tq_status tq_attend(const tq_params* kp, const tq_params* vp, const float* q, int segs,
                    int group, tq_cache keys, tq_cache vals, const int32_t* len, int64_t T,
                    float scale, float* out, void* ws, size_t ws_bytes, void* stream);

/* The two parts of tq_attend, for callers that overlap the query side with
 * other work (a decode step can prepare the new queries on a second stream
 * while it appends the step's keys and values, which the pack does not
 * read): tq_attend_prepare writes the query pack of every segment into ws
 * (kp, q, segs, group and ws as for tq_attend; ws_bytes at least the pack's
 * share, which tq_attend_workspace covers); tq_attend_prepared runs the rest
 * of tq_attend against the pack ws holds, from the last tq_attend_prepare
 * with the same kp, segs and group on this workspace (other arguments as for
 * tq_attend).  A prepare must not run while an attention that reads the same
 * workspace is still in flight.  The result equals tq_attend's. */
tq_status tq_attend_prepare(const tq_params* kp, const float* q, int segs, int group, void* ws,
                            size_t ws_bytes, void* stream);
tq_status tq_attend_prepared(const tq_params* kp, const tq_params* vp, int segs, int group,
                             tq_cache keys, tq_cache vals, const int32_t* len, int64_t T,
                             float scale, float* out, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes tq_scores_topk needs. */
size_t tq_scores_topk_workspace(const tq_params* kp, int nq, int64_t T, int k);

/* Top-k retrieval by the asymmetric estimator (the estimator of tq_scores) over
 * T prod records 0..T-1 encoded at d_rot = 2048 with the sign-flipped Hadamard
 * rotation (tq_encode_prod_ws), for nq queries.  With kp->s == NULL the records
 * are MSE-only (tq_encode_mse at d_rot = 2048) and the estimate is the MSE
 * inner product n_t <rot(q), c[idx_t]> (b index bits, b = 1..4):
 *   idx[i][0..k)  record indices of the k largest s(q_i, t), best first,
 *                 ties to the lower index (int64, device)
 *   val[i][0..k)  those estimates (float32, device)
 * q       device f32 [nq][d], d a multiple of 4, zero-padded to 2048
 * keys    record t at keys.planes + t * record words (seg_stride unused)
 * ws      device workspace of tq_scores_topk_workspace() bytes, 256-B aligned
 * Supported: 1 <= k <= 16, T >= k; prod keys with b = 2, 3 or 4 bits and
 * m = 2048 or 1024 QJL rows (kappa = sqrt(pi/2) / m).
 * Launches: query transform, projection GEMM and quantisation; per block of
 * 65536 records the bit-plane score GEMM and a per-query top-k; a final merge. */
tq_status tq_scores_topk(const tq_params* kp, const float* q, int nq, tq_cache keys, int64_t T, int k,
                         int64_t* idx, float* val, void* ws, size_t ws_bytes, void* stream);

/* ---- PolarQuant as stage 1 -------------------------------------------------
 * The FastVQ README ("PolarQuant Algorithm"; its "Implementation Notes" name
 * the paper's transform as the full recursive one, which this is; its
 * "TurboQuant Combination" for the optional QJL stage).
 *
 * With n = ||x||, u = x / n (0 for x = 0) and y = rot(u) (d = d_rot = 2^L):
 *   level 1      psi = atan2(y[2j+1], y[2j]) in (-pi, pi] for each coordinate
 *                pair, rho = the pair's length (j = 0 .. d/2 - 1)
 *   level l > 1  psi = atan2(rho[2j+1], rho[2j]) in [0, pi/2] over the lengths
 *                of level l - 1, rho = their combined length
 *   level L leaves one length, ||y|| = 1: the record keeps n and d - 1 codes.
 * Each angle's code is the number of its level's boundaries at or below it
 * (Lloyd-Max cells of the angle's law after a uniform rotation: uniform at
 * level 1, sin^2 psi ~ Beta(2^(l-2), 2^(l-2)) above; tq_build_polar_codebook).
 * The reconstruction y~ splits the unit length down the levels with the
 * centroid angles (rho cos, rho sin), so ||y~|| = 1, and x~ = n rot^T(y~).
 * With m = d the QJL stage follows on r = y - y~ (z = [S r >= 0], gamma = ||r||),
 * and the score estimate is
 *   s(q, t) = n_t ( <rot(q), y~_t> + gamma_t sqrt(pi/2)/m <S rot(q), 2 z_t - 1> ).
 *
 * Record (u32 words, then float16 scalars in their own array):
 *   level-1 stream  d/2 codes of bits1 bits, code j at bits j*bits1 .. of a
 *                   little-endian bit stream (bit k in bit k%32 of word k/32):
 *                   d*bits1/64 words
 *   upper stream    the d/2 - 1 codes of levels 2 .. L, level by level and in
 *                   ascending position, bits each, same packing:
 *                   ceil((d/2 - 1) bits / 32) words
 *   sign words      m/32 words of QJL bits (m > 0)
 *   scalars         float16 n, and float16 gamma when m > 0
 * At d = 128 that is 2 bits1 + 2 bits + m/32 words; planes [records][words],
 * scalars [records][1 or 2]; record r of segment s is s * seg_stride + t. */
typedef struct {
  int d;                    /* 128 */
  int rot;                  /* TQ_ROT_DENSE or TQ_ROT_HADAMARD (one round) */
  int bits1;                /* bits of each level-1 code, 1..4 */
  int bits;                 /* bits of each code at levels 2..L, 1..4 */
  int m;                    /* QJL rows: 0 (no second stage) or d */
  const float* pi;          /* device f32 [d][d] (dense; else NULL) */
  const float* eps;         /* device f32 [d] of +1/-1 (hadamard; else NULL) */
  const float* s;           /* device f32 [m][d] (m > 0; else NULL) */
  const float* centroids;   /* HOST f32: 2^bits1 level-1 centroids, then 2^bits for each level 2..L */
  const float* boundaries;  /* HOST f32: 2^bits1 - 1 level-1 boundaries, then 2^bits - 1 per level */
} tq_polar_params;
/* Codebook requirements (TQ_ERR_INVALID_ARG otherwise): finite centroids,
 * boundaries strictly between their neighbouring centroids; level-1
 * boundaries in (-pi, pi), upper-level boundaries in (0, pi/2). */

/* Lloyd-Max codebook of a level's angle (host, float64, deterministic):
 * level 1 the uniform grid of 2^bits cells from -pi; level >= 2 the Lloyd-Max
 * quantizer of the density proportional to sin^(2^(l-1) - 1)(2 psi) on
 * [0, pi/2], symmetric about pi/4 (explainer page section 5: midpoint
 * boundaries, conditional-mean centroids).  1 <= level <= 16, 1 <= bits <= 4.
 * centroids: host double[2^bits], boundaries: host double[2^bits - 1]. */
tq_status tq_build_polar_codebook(int level, int bits, double* centroids, double* boundaries);

/* Words per polar record (0 for invalid parameters). */
size_t tq_polar_record_words(const tq_polar_params* p);

/* PolarQuant encode of n vectors into polar records.
 * x, dtype, n, ld_x, slot: as for tq_encode_prod; out.planes u32
 * [records][tq_polar_record_words], out.scalars f16 [records][m ? 2 : 1],
 * out.records >= 1, a vector whose record lies outside [0, out.records) is
 * not written.  One launch: the rotation (and the QJL projection) on the
 * matrix cores in fp16 hi/lo parts, the transform and the codes per lane.
 * Supported: d = 128. */
tq_status tq_polar_encode(const tq_polar_params* p, const void* x, int dtype, int64_t n, int64_t ld_x,
                          tq_cache out, const int64_t* slot, void* stream);

/* Dequantize polar records 0 .. n-1 of `in`: out[i][0..d) = x~_i (float32,
 * device, rows ld_out >= d apart, 4-byte aligned).  The QJL bits, if any, are
 * not used (the reconstruction is stage 1's).  Needs n <= in.records. */
tq_status tq_polar_decode(const tq_polar_params* p, tq_cache in, int64_t n, float* out, int64_t ld_out,
                          void* stream);

/* Score estimates of query heads against polar keys (the formula above; the
 * first term alone when m = 0), in the shapes of tq_scores:
 * q device f32 [segs*group][d] (16-byte aligned), len device int32 [segs] or
 * NULL, scores device f32 [segs*group][T] (t >= len not written), keys with
 * (segs - 1) * seg_stride + T <= keys.records.  One launch; each workgroup
 * rotates and projects its segment's query heads and builds per-head tables
 * in the LDS (the level-1 pair terms per code, the QJL sign terms per nibble)
 * before streaming its tokens.  Supported: d = 128, 1 <= group <= 16. */
tq_status tq_polar_scores(const tq_polar_params* p, const float* q, int segs, int group, tq_cache keys,
                          const int32_t* len, int64_t T, float* scores, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
