/*
 * tq.h - C ABI of libtq: TurboQuant-style KV-cache compression and decode attention
 * computed directly over the compressed cache, for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources are the public web pages on the method):
 *  - Compression (TurboQuant page, de.news.hada.io/topic?id=27867, "Funktionsweise von
 *    TurboQuant", steps 1 and 2; TurboQuant explainer, chatgpz.de, "Stufe 1" and
 *    "Stufe 2"): a seeded random rotation Pi, a fixed Lloyd-Max code for N(0,1) applied to
 *    every rotated coordinate z = (Pi k) * sqrt(d) / |k| (Hacker News comments on the
 *    TurboQuant page), and a 1-bit QJL sign sketch of the key residual
 *    ("QJL: Eine 1-Bit-Methode ohne Overhead").  Values get codes only.
 *  - Decode attention over the compressed cache: inner products estimated from the codes
 *    and signs, softmax, value aggregation in the rotated basis, optional exact ("hot")
 *    tokens in the same softmax (Monarch v3 page, "Wie es funktioniert").
 *  - Self-Indexing top-k (Self-Indexing KVCache page, gist.science 2603.14224,
 *    "Methodologie" 1-3): 1-bit sign patterns of 4-dim groups after channel-mean
 *    centring, 16 centroids per group, LUT-GEMV scores, top-k.
 *  - Bulk scan: estimates for many queries against a whole compressed cache
 *    (TurboQuant page, "Leistung bei der Vektorsuche").
 *
 * Conventions
 *  - Every entry point returns tq_status.  TQ_OK = 0.  On any other status nothing was
 *    enqueued and no output was written; tq_last_error() gives a thread-local message.
 *    Shapes, dtypes, bit widths, alignment and null pointers are validated on the host
 *    before any launch.  A failing launch returns TQ_ERR_DEVICE.  Faults during
 *    asynchronous execution surface at the caller's next stream synchronisation.
 *  - Tensors are caller-owned DEVICE pointers unless a parameter says "host".  Work is
 *    enqueued on the caller's hipStream_t (NULL = the default stream); the library never
 *    synchronises the host and never allocates or frees device memory outside
 *    tq_create/tq_destroy.  Calls that take a workspace need
 *    tq_*_workspace_size() bytes of device memory, 256-byte aligned.
 *  - A handle is immutable after tq_create, so concurrent calls on different streams
 *    are allowed.  Calls that share a workspace or output buffer must be ordered.
 *  - A TQ_KEY_POLAR handle is accepted by tq_compress_kv, tq_decode_workspace_size,
 *    tq_decode_attention, tq_decode_attention_noalloc, tq_scan_workspace_size,
 *    tq_score_scan, tq_record_bytes, the hot/cold step, tq_sparse_attention and the
 *    sign-index / top-k calls (which read raw keys); tq_debug_quantize (scalar codes from
 *    given rotated coordinates) returns TQ_ERR_UNSUPPORTED for it.
 *  - Inputs must be finite.  Non-finite inputs give unspecified codes and outputs but
 *    never an out-of-bounds access.
 *
 * Record layout (one contiguous record per token per KV head, little-endian).  Every field
 * starts on a 32-bit word; padding bytes are zero:
 *    [ key codes  : KB = 4 * ceil(head_dim * key_bits / 32) bytes                   ]
 *    [ QJL signs  : qjl_dim / 8 bytes  (stream bit j = 1 iff (S e)_j >= 0)           ]
 *    [ value codes: VB = 4 * ceil(head_dim * value_bits / 32) bytes                 ]
 *    [ r_k float32 | rho float32 | r_v float32 ]
 *    [ zero pad to a multiple of 16 bytes ]
 *  so record_bytes = 16 * ceil((KB + qjl_dim / 8 + VB + 12) / 16) (tq_record_bytes); e.g.
 *  head_dim 128, 3-bit keys, qjl_dim 128, 4-bit values: 48 + 16 + 64 + 12 -> 144 bytes.
 *  1-, 2- and 4-bit code fields and the sign field are little-endian bitstreams: code i occupies
 *  stream bits [b*i, b*i + b), stream bit n being bit n % 8 of byte n / 8.
 *  3-bit code fields are groups of 32 codes; group g is the 12 bytes at 12 g, read as
 *  little-endian 32-bit words W0, W1, W2.  Code j < 24 of a group occupies bits
 *  [8 (j % 4) + 3 floor((j % 8) / 4), +3) of W_floor(j / 8).  Code 24 + r (r < 8) is bits
 *  [3 floor(r / 4), +3) of the 6-bit value T_k of byte lane k = r % 4, where bit t of T_k is
 *  bit 8 k + 6 + (t % 2) of W_floor(t / 2).  (Masking a word with 0x07070707, or shifting it by
 *  3 and masking, gives four codes, one per byte.)  When head_dim is not a multiple of 32 the
 *  last head_dim % 32 codes follow the whole groups as a plain 3-bit bitstream (head_dim 200:
 *  6 groups of 72 bytes, then codes 192..199 in 3 bytes, padded to 76 bytes).
 *  Polar key codes (TQ_KEY_POLAR) replace the key code field by
 *    [ level-1 angle codes: (head_dim/2) * key_bits / 8 bytes, a key_bits-bit bitstream ]
 *    [ codes of levels 2..L, level 2 first, node order: a polar_upper_bits-bit bitstream
 *      in 4 * ceil((head_dim/2 - 1) * polar_upper_bits / 32) bytes ]
 *  A cache is an array records[batch][kv_heads][capacity][record_bytes].
 *  Sign index: one record of head_dim/8 bytes per token per KV head; the 4-bit pattern of
 *  channel group g (channels 4g..4g+3, bit j = channel 4g+j) sits at stream bits
 *  [4g, 4g+4).  Index array: index[batch][kv_heads][capacity][head_dim/8];
 *  codebook[batch][kv_heads][head_dim/4][16][4] float32; mean[batch][kv_heads][head_dim].
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tq_status {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARGUMENT = 1,   /* bad pointer, shape, stride, dtype or value        */
  TQ_ERR_UNSUPPORTED = 2,        /* valid but not built (e.g. polar keys at head_dim 200) */
  TQ_ERR_WORKSPACE_TOO_SMALL = 3,
  TQ_ERR_OUT_OF_MEMORY = 4,      /* tq_create only                                   */
  TQ_ERR_DEVICE = 5              /* a HIP call or kernel launch failed               */
} tq_status;

typedef enum tq_dtype { TQ_F32 = 0, TQ_F16 = 1, TQ_BF16 = 2 } tq_dtype;

/* Stage-1 key codec.  TQ_KEY_SCALAR: a Lloyd-Max code per rotated coordinate.
 * TQ_KEY_POLAR: the PolarQuant variant (TurboQuant page, section "PolarQuant"): the rotated
 * key y = Pi k is taken in coordinate pairs; each pair becomes a radius and an angle
 * atan2(y_2i+1, y_2i) in (-pi, pi]; the radii are paired again (angle atan2(right, left)
 * in [0, pi/2]) until one radius remains, so d = 2^L gives d - 1 angles on L levels.
 * Level-1 angles are coded on a uniform grid of 2^key_bits cells from -pi (centres as
 * reconstruction values); level l >= 2 angles on the Lloyd-Max grid (2^polar_upper_bits
 * cells) of their exact law for a random direction, density proportional to
 * sin(2 psi)^(2^(l-1) - 1) on [0, pi/2].  code = #{j : angle >= bound_j} with the angle
 * in float64 and the float32 bounds; two zero inputs have angle 0.  The key is rebuilt as
 * r_k * u, u the unit vector of the grid angles; QJL then sketches e = y - r_k u. */
typedef enum tq_key_codec { TQ_KEY_SCALAR = 0, TQ_KEY_POLAR = 1 } tq_key_codec;

typedef struct tq_config {
  int32_t head_dim;       /* d: 64 or 128 for every call; any other multiple of 8 up
                             to 256 (scalar keys) for every call but the hot/cold step
                             (direct kernels that read d at run time), which returns
                             TQ_ERR_UNSUPPORTED for such a handle                      */
  int32_t key_bits;       /* b_k: bits per rotated key coordinate, 1..4; polar: bits
                             per level-1 angle, 2 or 4                                 */
  int32_t qjl_dim;        /* m: 0 (no QJL sketch) or a multiple of 32, at most 256     */
  int32_t value_bits;     /* b_v: 1..4                                                 */
  uint64_t rotation_seed; /* seed of the Gaussian matrix whose QR factor is Pi         */
  uint64_t qjl_seed;      /* seed of the QJL projection S                              */
  int32_t key_codec;      /* tq_key_codec (0 = scalar)                                 */
  int32_t polar_upper_bits; /* polar: bits per angle above level 1: 1, 2 or 4; else 0  */
} tq_config;

typedef struct tq_handle tq_handle;

/* Message of the last failing call on this thread ("" if none).  Never NULL. */
const char* tq_last_error(void);

/* Build the handle's constants on the host and upload them to the current device.
 *  - Pi (d x d): Q factor of a d x d Gaussian matrix G drawn from rotation_seed, with the
 *    signs of Q's columns chosen so that R = Q^T G has a positive diagonal, rounded to
 *    float32 (TurboQuant page, "Funktionsweise", step 1: random rotation).
 *  - S (m x d): i.i.d. N(0,1) from qjl_seed, float32 (TurboQuant page, "QJL").
 *  - Lloyd-Max levels/boundaries for N(0,1) at key_bits and value_bits, iterated in
 *    float64 and rounded to float32 (Hacker News comments on the TurboQuant page).
 *  Gaussians: SplitMix64 (Steele, Lea, Flood 2014) word i of a seed is
 *  mix(seed + (i+1) * 0x9E3779B97F4A7C15); pair k of normals is Box-Muller of words 2k,
 *  2k+1 with u1 = ((w>>11)+1)*2^-53, u2 = (w>>11)*2^-53.  Matrices are filled row-major.
 *  The only call that allocates device memory.  *out receives the handle. */
tq_status tq_create(const tq_config* cfg, tq_handle** out);
tq_status tq_destroy(tq_handle* h);

/* Host-only: the constants tq_create would build, written to HOST arrays (any may be
 * NULL): pi[d*d], s[m*d], key_levels[2^kb], key_bounds[2^kb - 1], value_levels[2^vb],
 * value_bounds[2^vb - 1].  Needs no GPU. */
tq_status tq_host_constants(const tq_config* cfg, float* pi, float* s, float* key_levels,
                            float* key_bounds, float* value_levels, float* value_bounds);

/* Host-only: the polar angle grids tq_create would build for a TQ_KEY_POLAR config,
 * written to HOST arrays levels[L][16] and bounds[L][16] (L = log2 head_dim; row l-1 is
 * level l; entries past 2^bits levels / 2^bits - 1 bounds are left untouched).  Row 0 is
 * the uniform grid of key_bits; rows 1.. the Lloyd-Max grids of polar_upper_bits, iterated
 * in float64 (cell mass and first moment by composite Gauss-Legendre quadrature) until
 * the levels move less than 1e-13, rounded to float32.  Needs no GPU. */
tq_status tq_polar_host_constants(const tq_config* cfg, float* levels, float* bounds);

/* Bytes of one cache record and of one sign-index record (host pointers). */
tq_status tq_record_bytes(const tq_handle* h, size_t* record_bytes, size_t* index_record_bytes);

/* Compress keys and values into records (TurboQuant page, "Funktionsweise", steps 1-2).
 *  k, v: element (b, t, h, i) at k[b*seq_stride + t*tok_stride + h*head_stride + i] in
 *  dtype dt (strides in elements; the innermost dimension is contiguous).
 *  Writes records[b][h][first_slot + t] for t < n_tokens, b < batch, h < kv_heads;
 *  requires first_slot + n_tokens <= capacity.  Per token-head: r = |k|;
 *  x = Pi k, z = x * sqrt(d) / r (z = 0 when r = 0), code c_i = #{j : z_i >= tau_j}
 *  (float32 comparison); residual e = x - (r/sqrt(d)) gamma[c]; rho = |e|; QJL bit j =
 *  [(S e)_j >= 0].  Polar keys: angles and codes as tq_key_codec states, e = x - r u.
 *  Values: codes and r_v only.  The rotation and projection run as
 *  float64 matrix-core (MFMA) products, so codes equal a float64 reference except where
 *  a rotated coordinate lies within rounding of a boundary. */
tq_status tq_compress_kv(const tq_handle* h, const void* k, const void* v, tq_dtype dt,
                         int32_t batch, int64_t n_tokens, int32_t kv_heads,
                         int64_t seq_stride, int64_t tok_stride, int64_t head_stride,
                         void* records, int64_t capacity, int64_t first_slot,
                         hipStream_t stream);

/* Test entry: records from given rotated inputs (device float32 arrays):
 *  z_k[n][d], z_v[n][d] (already scaled by sqrt(d)/r), p[n][m] (S e), r_k[n], rho[n],
 *  r_v[n].  Codes are c = #{j : z >= tau_j}, bits [p >= 0].  Writes records[n]. */
tq_status tq_debug_quantize(const tq_handle* h, const float* z_k, const float* p,
                            const float* r_k, const float* rho, const float* z_v,
                            const float* r_v, int64_t n, void* records, hipStream_t stream);

/* Decode attention over the compressed cache.
 *  q[b][hq][d] (dtype q_dt); KV head of query head hq is hq / (q_heads / kv_heads).
 *  Cold tokens of sequence b: slots [0, seq_lens[b]) of records[b][h] (seq_lens: device
 *  int32[batch], each <= capacity), or, in gather mode (sel_idx != NULL), the slots
 *  sel_idx[b][h][0..k_sel) that are >= 0 (device int32; -1 entries are skipped; each
 *  slot < capacity).  Cold logit = scale * s_t with
 *    s_t = (r_k/sqrt(d)) <Pi q, gamma_k[c_t]> + sqrt(pi/2)/m rho_t <S Pi q, 2 bit_t - 1>
 *  (the QJL estimator; the second term is absent when m = 0).  Polar keys: the first
 *  term is r_k <Pi q, u_t>, u_t the unit vector of the token's grid angles.
 *  Exact segment (optional, hot_lens != NULL): hot_k/hot_v[b][h][hot_capacity][d] in
 *  hot_dt (each pointer aligned to 8 elements), tokens [0, hot_lens[b]);
 *  logit = scale * <q, k>; one softmax over cold+hot
 *  (Monarch v3 page, "Wie es funktioniert").  scale = 0 selects 1/sqrt(d).
 *  out[b][hq][d] float32 = (Pi^T sum_cold p_t vhat_t + sum_hot p_t v_t) / sum_t p_t,
 *  vhat_t = (r_v/sqrt(d)) gamma_v[c^v_t]; zero when no token is attended.
 *  lse[b][hq] (optional) = log sum_t exp(logit_t) (-inf when empty).
 *  logits (optional, for tests) float32 [b][hq][n_cold_max + hot_capacity], n_cold_max =
 *  capacity (or k_sel in gather mode); cold logits first, then hot; unattended entries are
 *  not written.  workspace: tq_decode_workspace_size bytes. */
tq_status tq_decode_workspace_size(const tq_handle* h, int32_t batch, int32_t q_heads,
                                   int32_t kv_heads, int64_t capacity, int32_t k_sel,
                                   size_t* bytes);
tq_status tq_decode_attention(const tq_handle* h, const void* q, tq_dtype q_dt, int32_t batch,
                              int32_t q_heads, int32_t kv_heads, const void* records,
                              int64_t capacity, const int32_t* seq_lens,
                              const void* hot_k, const void* hot_v, tq_dtype hot_dt,
                              const int32_t* hot_lens, int64_t hot_capacity,
                              const int32_t* sel_idx, int32_t k_sel, float scale, float* out,
                              float* lse, float* logits, void* workspace, size_t ws_bytes,
                              hipStream_t stream);

/* tq_decode_attention without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Arguments, outputs and errors as tq_decode_attention.  The call allocates nothing: its
 * scratch is one fixed device array of 16 MiB (16 << 20 bytes) per GPU, built into the
 * library and held until the process ends; tq_create looks up its address on the handle's
 * device.  A decode whose tq_decode_workspace_size exceeds 16 MiB returns
 * TQ_ERR_WORKSPACE_TOO_SMALL with nothing enqueued.  Every call on a GPU shares that GPU's
 * array (nothing in it needs to start at zero): calls that may overlap on one GPU - on
 * different streams, or from different threads - race and must be ordered by the caller. */
tq_status tq_decode_attention_noalloc(const tq_handle* h, const void* q, tq_dtype q_dt,
                                      int32_t batch, int32_t q_heads, int32_t kv_heads,
                                      const void* records, int64_t capacity,
                                      const int32_t* seq_lens, const void* hot_k,
                                      const void* hot_v, tq_dtype hot_dt, const int32_t* hot_lens,
                                      int64_t hot_capacity, const int32_t* sel_idx, int32_t k_sel,
                                      float scale, float* out, float* lse, float* logits,
                                      hipStream_t stream);

/* Self-Indexing sign index of keys over slots [first_slot, first_slot + n_tokens)
 * (Self-Indexing page, "Methodologie" 1-2).  k addressed as in tq_compress_kv.
 * mean[b][h][i] = float32(mean_t k), bit = [k >= mean] (float32), pattern per 4-channel
 * group, codebook[b][h][g][p][0..3] = float32 mean of (k - mean) over members (0 if none).
 * The mean and centroids use only the tokens of this call.  workspace:
 * tq_index_workspace_size bytes. */
tq_status tq_index_workspace_size(const tq_handle* h, int32_t batch, int32_t kv_heads,
                                  size_t* bytes);
tq_status tq_build_sign_index(const tq_handle* h, const void* k, tq_dtype dt, int32_t batch,
                              int64_t n_tokens, int32_t kv_heads, int64_t seq_stride,
                              int64_t tok_stride, int64_t head_stride, void* index,
                              float* codebook, float* mean, int64_t capacity,
                              int64_t first_slot, void* workspace, size_t ws_bytes,
                              hipStream_t stream);

/* Top-k tokens per (sequence, KV head) from the sign index (Self-Indexing page,
 * "Methodologie" 3: LUT-GEMV).  Table LUT[g][p] = ((q0 c0 + q1 c1) + q2 c2) + q3 c3 in
 * float64 for each query head of the group; s = largest integer with
 * G * (d/4) * max|LUT| * 2^s <= 2^30 (s = 0 if max|LUT| = 0); entries rounded half to
 * even to integers; score_t = sum over heads and groups (int32, exact).  Ranking: score
 * descending, then token index ascending.  out_idx[b][h][k] = the min(k, n) chosen slots
 * in ascending order, -1 padded; out_count[b][h] = min(k, n); out_scores (optional)
 * [b][h][k] = their scores (0 padded).  n = seq_lens[b] (device int32).  k >= 0.
 * workspace: tq_select_workspace_size bytes. */
tq_status tq_select_workspace_size(const tq_handle* h, int32_t batch, int32_t kv_heads,
                                   int64_t capacity, size_t* bytes);
tq_status tq_select_topk(const tq_handle* h, const void* q, tq_dtype q_dt, int32_t batch,
                         int32_t q_heads, int32_t kv_heads, const void* index,
                         const float* codebook, int64_t capacity, const int32_t* seq_lens,
                         int32_t k, int32_t* out_idx, int32_t* out_count, int32_t* out_scores,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

/* Sparse attention in one call (Self-Indexing page, "Methodologie" 3-5: select from the
 * sign index, then attend to the selected tokens' compressed keys and values).  out / lse as
 * tq_decode_attention(q, records, seq_lens, exact segment, sel_idx = the out_idx that
 * tq_select_topk(q, index, codebook, seq_lens, k) returns, scale): the same top-k set (same
 * ranking and tie rule), the same estimator, one softmax with the optional exact segment
 * (hot_k / hot_v / hot_lens, e.g. always-attended sink tokens); scalar or polar key codes.
 * The selected indices are not written out.  Requires qjl_dim in {0, 32, 64, 96, 128} and at most 16 query heads per
 * KV head.  workspace: tq_sparse_workspace_size bytes (256-byte aligned).  Nothing is
 * allocated; the host is not synchronised. */
tq_status tq_sparse_workspace_size(const tq_handle* h, int32_t batch, int32_t q_heads,
                                   int32_t kv_heads, int64_t capacity, size_t* bytes);
tq_status tq_sparse_attention(const tq_handle* h, const void* q, tq_dtype q_dt, int32_t batch,
                              int32_t q_heads, int32_t kv_heads, const void* index,
                              const float* codebook, const void* records, int64_t capacity,
                              const int32_t* seq_lens, int32_t k, const void* hot_k,
                              const void* hot_v, tq_dtype hot_dt, const int32_t* hot_lens,
                              int64_t hot_capacity, float scale, float* out, float* lse,
                              void* workspace, size_t ws_bytes, hipStream_t stream);

/* Bulk scan (TurboQuant page, "Leistung bei der Vektorsuche"): for q[b][h][i][d]
 * (i < n_queries) and every slot t < n_tokens of records[b][h], scores[b][h][i][t] =
 * s_t as in tq_decode_attention (unscaled estimate, no softmax; polar keys included).
 * float32 output.  At head_dim 128 with 2/3-bit scalar keys and m in {0, 128} the products
 * are exact int32 limb products; elsewhere fp16 hi + lo matrix-core products of operands
 * scaled to their row maxima (error ~2^-22 of sum_k |q_k t_k|).  workspace:
 * tq_scan_workspace_size bytes. */
tq_status tq_scan_workspace_size(const tq_handle* h, int32_t batch, int32_t kv_heads,
                                 int32_t n_queries, size_t* bytes);
tq_status tq_score_scan(const tq_handle* h, const void* q, tq_dtype q_dt, int32_t batch,
                        int32_t kv_heads, int32_t n_queries, const void* records,
                        int64_t capacity, int64_t n_tokens, float* scores, void* workspace,
                        size_t ws_bytes, hipStream_t stream);

/* Measurement support: on this thread, the next tq_decode_attention, tq_compress_kv,
 * tq_select_topk, tq_sparse_attention or tq_score_scan call records `start` on its stream just before its main
 * kernel (decode: the split-K scan; compress: the compress kernel; select: the sign-index
 * score kernel; scan: the score kernel) and `stop` just after it, then forgets both.
 * Events are caller-created (hipEventCreate) and caller-owned; NULL, NULL clears. */
tq_status tq_set_profile_events(hipEvent_t start, hipEvent_t stop);

/* Hot/cold decode step (Monarch v3 page, "Wie es funktioniert" and its decode loop; the
 * choices the page leaves open are stated here).  Per sequence b the state holds:
 *  - a hot ring: hot_k/hot_v[b][h][hot_capacity][head_dim] in hot_dt, hot_len[b] exact tokens
 *    from ring slot hot_start[b] (oldest first); hot_len[b] <= window before each step;
 *  - a cold region: records[b][h][cold_capacity] (tq_compress_kv layout), cold_len[b] tokens,
 *    hits[b][cold_capacity] consecutive qualifying steps per cold token, overflow[b] set to 1
 *    once an eviction found the cold region full (those tokens were dropped).
 * One step, for queries q[b][hq][d] and the step's token k_new/v_new[b][h][d] (hot_dt):
 *  1. the step's token joins the ring (newest);
 *  2. query head hq reads the cold tokens iff scale * max_t <q, k_t> over the ring is below
 *     cfg->cold_gate (+inf: always, and the ring logits are then not formed for the gate); out /
 *     lse = attention over the ring plus, for open heads,
 *     the cold tokens (TurboQuant estimator, as tq_decode_attention), one softmax;
 *  3. a cold token whose weight p (maximum over the open heads) is >= cfg->promote_weight
 *     counts one more consecutive step, else its count resets; at cfg->promote_steps (0: never)
 *     it is promoted: k = Pi^T (r_k/sqrt(d)) gamma_k[c] (polar keys: k = Pi^T (r_k u), u the
 *     unit vector of the grid angles), v = Pi^T (r_v/sqrt(d)) gamma_v[c_v]
 *     (float64, rounded to hot_dt) join the ring as its newest tokens in ascending cold order,
 *     and the cold slots are freed by moving the last cold token into each, highest slot first;
 *  4. while the ring holds more than cfg->window tokens, its oldest are compressed (float64
 *     rotation, scalar or polar key codes as tq_compress_kv) and appended to the cold region
 *     with count 0.
 * hot_capacity must be >= window + 1 + floor(1 / promote_weight) * q_heads (when promotion is
 * on).  gate_out (optional, [b][hq]) receives the step-2 decisions; lse is optional.
 * workspace: tq_monarch_workspace_size bytes.  All state stays on the device; the host is
 * never synchronised. */
typedef struct {
  int32_t window;          /* hot tokens kept per sequence after each step */
  float cold_gate;         /* a head reads the cold tokens iff its best hot logit is below this */
  float promote_weight;    /* attention weight a cold token needs in a step (e.g. 0.15) */
  int32_t promote_steps;   /* consecutive such steps before promotion (e.g. 3; 0 = never) */
} tq_monarch_config;

typedef struct {
  void* hot_k;
  void* hot_v;
  tq_dtype hot_dt;
  int64_t hot_capacity;
  int32_t* hot_start;
  int32_t* hot_len;
  void* records;
  int64_t cold_capacity;
  int32_t* cold_len;
  int32_t* hits;
  int32_t* overflow;
} tq_monarch_state;

tq_status tq_monarch_workspace_size(const tq_handle* h, int32_t batch, int32_t q_heads,
                                    int32_t kv_heads, int64_t hot_capacity, int64_t cold_capacity,
                                    size_t* bytes);
tq_status tq_monarch_step(const tq_handle* h, const tq_monarch_config* cfg,
                          const tq_monarch_state* state, const void* q, tq_dtype q_dt,
                          int32_t batch, int32_t q_heads, int32_t kv_heads, const void* k_new,
                          const void* v_new, float scale, float* out, float* lse,
                          int32_t* gate_out, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Measurement support: enqueue a streaming read of buf[0, bytes) (device memory, 16-byte
 * aligned, bytes a multiple of 16) that folds the data into sink (device uint32, at least
 * 64 x the device's compute-unit count words: one per wave, their XOR is the XOR of every
 * 32-bit word of the buffer).  The bench times it with
 * tq_set_profile_events to obtain its own HBM read ceiling.  Nothing else in the library
 * depends on it. */
tq_status tq_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
