// Internal declarations shared by the host runtime (tq_host.cpp) and the gfx950 kernels
// (tq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "../../include/tq.h"

namespace tq {

constexpr int kMaxLevels = 16;   // 2^4: key/value codes have at most 4 bits

// Optional events recorded around the main kernel of one call (measurement only).
struct ProfileEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  void before(hipStream_t s) const { if (start) (void)hipEventRecord(start, s); }
  void after(hipStream_t s) const { if (stop) (void)hipEventRecord(stop, s); }
};
constexpr int kWave = 64;

// Per-handle constants passed by value to every kernel.
struct Consts {
  float key_levels[kMaxLevels];
  float key_bounds[kMaxLevels];   // 2^kb - 1 used
  float val_levels[kMaxLevels];
  float val_bounds[kMaxLevels];   // 2^vb - 1 used
  int d, kb, m, vb;
  int kbytes, sbytes, vbytes;     // code / sign field sizes in bytes
  int rec_bytes;                  // record stride in bytes (multiple of 16)
  int norm_off;                   // byte offset of r_k (then rho, r_v)
  float inv_sqrt_d;               // 1/sqrt(d) rounded to float32
  double sqrt_d;                  // sqrt(d) in float64
  float qjl_coef;                 // sqrt(pi/2)/m rounded to float32 (0 when m = 0)
  float key_fix;                  // fixed-point scale of the key levels for integer products:
                                  // |level| * key_fix <= 32512, levels * key_fix near integers
  float key_fix3;                 // three-limb scale: max |level| * key_fix3 = 127 * 65536
  // polar key codes (0 / unused for the scalar codec)
  int polar;                      // 1: keys are recursive polar angle codes
  int pb1, pbh;                   // bits per level-1 angle / per higher angle
  int plevels;                    // L = log2 d
  int l1_bytes;                   // bytes of the level-1 code stream (the rest of kbytes: levels 2..L)
};

constexpr int kMaxPolarLevels = 8;   // log2 of the largest head_dim (128) is 7

// Polar angle tables in device memory, row l-1 = level l, 16 entries per row:
//   bounds  float  [8][16]  (unused entries +inf)
//   cs64    double [8][16][2]  cos, sin of the float32 grid levels (float64)
//   cs32    float  [8][16][2]  the same rounded to float32
struct PolarTables {
  const float* bounds;
  const double* cs64;
  const float* cs32;
};

// Device buffers a handle owns.
struct DevConsts {
  const float* pi;        // [d][d] row-major (x = Pi k)
  const float* pi_t;      // Pi transposed, [d][d] row-major (row k = column k of Pi)
  const float* s_pi;      // S Pi ([m][d], float64 product rounded to float32): q_s = (S Pi) q
  const float* s;         // [m][d] row-major
  const float* s_t;       // S transposed, [d][m] row-major
  const float* pi_mfma;   // Pi in the order the compress kernel's MFMA A operand reads it
  const float* s_mfma;    // S in the same order
  PolarTables polar;      // polar key codec only (null pointers otherwise)
};

// ---- launchers (tq_kernels.hip) ----------------------------------------------------------
hipError_t launch_compress(const Consts& c, const DevConsts& dc, const void* k, const void* v,
                           tq_dtype dt, int batch, int64_t n_tokens, int heads,
                           int64_t seq_stride, int64_t tok_stride, int64_t head_stride,
                           void* records, int64_t capacity, int64_t first_slot,
                           hipStream_t stream, const ProfileEvents& ev);

hipError_t launch_debug_quantize(const Consts& c, const float* z_k, const float* p,
                                 const float* r_k, const float* rho, const float* z_v,
                                 const float* r_v, int64_t n, void* records,
                                 hipStream_t stream);

struct DecodePlan {
  int chunk;        // tokens per split-K chunk
  int n_chunks;
  int group;        // q_heads / kv_heads
  int hpl;          // heads per lane (1 or 4)
  bool key_pairs;   // key LUT indexed by pairs of codes (else single codes)
  bool sign_bytes;  // QJL LUT indexed by bytes (else nibbles)
  bool mfma;        // matrix-core scan (head_dim 128, 4 query heads per KV head)
  bool small;       // direct scan for short caches (chunks of at most 64 tokens)
  bool generic;     // head_dim other than 64 / 128: the generic direct kernel and merge
  size_t lds_bytes;
  size_t ws_qx, ws_qs, ws_part, ws_bop, ws_total;   // workspace offsets / size
};

bool plan_decode(const Consts& c, int batch, int q_heads, int kv_heads, int64_t n_max,
                 DecodePlan* plan);

// Extra inputs of a decode inside a hot/cold step: per-head gates and a ring-buffered hot
// region holding hot_lens[b] + hot_add tokens from slot hot_start[b].
struct DecodeHooks {
  const int32_t* gate;       // [B][Hq]
  const int32_t* hot_start;  // [B]
  int hot_add;
  // [B][capacity] float bits, zeroed: each open head's merge folds exp(logit - lse) of every
  // cold token into the per-token maximum (NULL: not formed)
  uint32_t* promo_w;
};
hipError_t launch_decode(const Consts& c, const DevConsts& dc, const DecodePlan& plan,
                         const void* q, tq_dtype q_dt, int batch, int q_heads, int kv_heads,
                         const void* records, int64_t capacity, const int32_t* seq_lens,
                         const void* hot_k, const void* hot_v, tq_dtype hot_dt,
                         const int32_t* hot_lens, int64_t hot_capacity,
                         const int32_t* sel_idx, int k_sel, float scale, float* out, float* lse,
                         float* logits, void* workspace, hipStream_t stream,
                         const ProfileEvents& ev, const DecodeHooks* hooks = nullptr);

struct IndexPlan {
  int chunk, n_chunks;
  size_t ws_mean, ws_csum, ws_ccnt, ws_total;
};
IndexPlan plan_index(const Consts& c, int batch, int heads, int64_t n_tokens);
hipError_t launch_sign_index(const Consts& c, const IndexPlan& plan, const void* k, tq_dtype dt,
                             int batch, int64_t n_tokens, int heads, int64_t seq_stride,
                             int64_t tok_stride, int64_t head_stride, void* index,
                             float* codebook, float* mean, int64_t capacity, int64_t first_slot,
                             void* workspace, hipStream_t stream);

struct SelectPlan {
  int n_chunks;                 // 4096-token chunks of the capacity
  size_t ws_lut, ws_scores, ws_hist, ws_cand, ws_chunk_cand, ws_chunk_above, ws_chunk_off, ws_params, ws_total;
};
SelectPlan plan_select(const Consts& c, int batch, int heads, int64_t capacity);

struct SparsePlan {
  SelectPlan select;
  size_t ws_select, ws_qx, ws_qs, ws_part, ws_total;
};
SparsePlan plan_sparse(const Consts& c, int batch, int q_heads, int kv_heads, int64_t capacity);
// Query prep (q_x = Pi q, q_s = S q_x for `rows` query rows) that launch_select may run in the
// same launch as its table build.
struct QueryPrep {
  const float* pi;
  const float* s;
  int m, rows;
  float* qx;
  float* qs;
};
hipError_t launch_select(const Consts& c, const SelectPlan& plan, const void* q, tq_dtype q_dt,
                         int batch, int q_heads, int kv_heads, const void* index,
                         const float* codebook, int64_t capacity, const int32_t* seq_lens,
                         int k, int32_t* out_idx, int32_t* out_count, int32_t* out_scores,
                         void* workspace, hipStream_t stream, const ProfileEvents& ev,
                         const QueryPrep* prep = nullptr, bool skip_exact = false);
hipError_t launch_sparse(const Consts& c, const DevConsts& dc, const SparsePlan& plan, const void* q,
                         tq_dtype q_dt, int batch, int q_heads, int kv_heads, const void* index,
                         const float* codebook, const void* records, int64_t capacity,
                         const int32_t* seq_lens, int k, const void* hot_k, const void* hot_v,
                         tq_dtype hot_dt, const int32_t* hot_lens, int64_t hot_capacity, float scale,
                         float* out, float* lse, void* workspace, hipStream_t stream,
                         const ProfileEvents& ev);

struct ScanPlan {
  bool mfma;        // matrix-core scan (head_dim 128, 2/3-bit keys, m in {0, 128})
  int n_groups;     // groups of 4 queries per (sequence, KV head) (matrix-core path: whole 16-query tiles)
  int kp;           // generic path: d + m rounded up to a multiple of 32
  size_t ws_q, ws_ql, ws_qscale, ws_total;
};
ScanPlan plan_scan(const Consts& c, int batch, int heads, int n_queries);
hipError_t launch_scan(const Consts& c, const DevConsts& dc, const ScanPlan& plan, const void* q,
                       tq_dtype q_dt, int batch, int heads, int n_queries, const void* records,
                       int64_t capacity, int64_t n_tokens, float* scores, void* workspace,
                       hipStream_t stream, const ProfileEvents& ev);

int stream_read_blocks();          // workgroups of the streaming read (256 threads each)
size_t stream_read_sink_words();   // one word per wave
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream,
                              const ProfileEvents& ev);

// Hot/cold step (tq_monarch_step).
struct MonarchPlan {
  DecodePlan decode;
  int64_t logit_stride;
  size_t ws_decode, ws_gate, ws_lse, ws_logits, ws_counts, ws_promo, ws_total;
};
struct MonarchStep {
  const void* q;
  tq_dtype q_dt;
  const void* k_new;
  const void* v_new;
  void* hot_k;
  void* hot_v;
  tq_dtype hot_dt;
  int64_t hot_cap, cold_cap;
  int32_t* hot_start;
  int32_t* hot_len;
  void* records;
  int32_t* cold_len;
  int32_t* hits;
  int32_t* overflow;
  float* out;
  float* lse;
  int32_t* gate_out;
  int batch, q_heads, kv_heads, window, promote_steps;
  float cold_gate, promote_weight, scale;
};
// Fixed device scratch of the allocation-free decode (tq_decode_attention_noalloc): one
// file-scope device array of kScratchBytes in the kernels' source file, so every GPU the
// library runs on holds its own copy until the process ends.  scratch_setup() looks up the
// array's address on the current device once (hipGetSymbolAddress) and keeps it per device;
// scratch_address(device) returns it (nullptr if setup never succeeded there).
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kScratchMaxDevices = 64;
hipError_t scratch_setup();
void* scratch_address(int device);

MonarchPlan plan_monarch(const Consts& c, int batch, int q_heads, int kv_heads, int64_t hot_cap,
                         int64_t cold_cap, bool* ok);
hipError_t launch_monarch_step(const Consts& c, const DevConsts& dc, const MonarchPlan& plan,
                               const MonarchStep& s, void* workspace, hipStream_t stream,
                               const ProfileEvents& ev);

}  // namespace tq
