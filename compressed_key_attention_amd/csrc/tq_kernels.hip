// gfx950 (MI355X) kernels of libtq.
//
//  compress_kernel       rotation and QJL projection as float64 MFMA products
//                        (v_mfma_f64_16x16x4f64), quantize/pack epilogue, one record per token
//  debug_quantize_kernel records from given rotated coordinates (same packing code)
//  query_prep_kernel     q_x = Pi q, q_s = S q_x (float64 accumulate)
//  decode_scan_kernel    split-K scan over packed records: LUT-GEMV key scores, online softmax,
//                        rotated-domain value aggregation; one partial (m, l, o_x) per chunk
//  decode_merge_kernel   log-sum-exp merge of the partials + exact segment + un-rotation
//  index_* kernels       Self-Indexing sign index (channel mean, patterns, centroids)
//  select_* kernels      integer LUT-GEMV scores, radix select, ordered compaction
//  compress_generic_kernel  the same at head_dims without a matrix-core layout (float64 loops)
//  scan_* kernels        bulk multi-query score scan (int8 matrix cores at head_dim 128; fp16
//                        hi / lo matrix-core products elsewhere)
//  polar_* helpers       the PolarQuant key codes (compress side) and their decode variants
//
// Method sources are cited at each kernel; the arithmetic each performs is stated there.

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "tq_internal.h"

namespace tq {

namespace {

constexpr float kNegInf = -INFINITY;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Load n (multiple of 8 for 16-bit types, of 4 for f32) consecutive elements starting at a
// 16-byte aligned address, converting to float32 (exact for bf16/f16/f32).
template <int N>
__device__ __forceinline__ void load_row(const void* base, tq_dtype dt, int64_t elem_off, bool valid,
                                         float (&out)[N]) {
  if (!valid) {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = 0.0f;
    return;
  }
  if (dt == TQ_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      uint4 u = p[i];
      out[4 * i + 0] = __uint_as_float(u.x);
      out[4 * i + 1] = __uint_as_float(u.y);
      out[4 * i + 2] = __uint_as_float(u.z);
      out[4 * i + 3] = __uint_as_float(u.w);
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      uint4 u = p[i];
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (dt == TQ_BF16) {
          out[8 * i + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
          out[8 * i + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
        } else {
          out[8 * i + 2 * j] = f16_bits_to_f32(w[j] & 0xFFFFu);
          out[8 * i + 2 * j + 1] = f16_bits_to_f32(w[j] >> 16);
        }
      }
    }
  }
}

__device__ __forceinline__ float load_elem(const void* base, tq_dtype dt, int64_t off) {
  if (dt == TQ_F32) return static_cast<const float*>(base)[off];
  const uint32_t b = static_cast<const uint16_t*>(base)[off];
  return dt == TQ_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// Code of a float32 coordinate: number of boundaries it reaches, c = #{j : z >= tau_j}.
// Unused boundary slots hold +inf.
// #{j : z >= bounds[j]} over the kMaxLevels - 1 = 15 ascending bounds (padded with +inf past
// the codebook's), by a four-step binary search: the same count as comparing all of them
__device__ __forceinline__ uint32_t quantize_code(float z, const float* bounds) {
  uint32_t c = 0;
  c += z >= bounds[c + 7] ? 8u : 0u;
  c += z >= bounds[c + 3] ? 4u : 0u;
  c += z >= bounds[c + 1] ? 2u : 0u;
  c += z >= bounds[c] ? 1u : 0u;
  return c;
}

// Append `nbits` low bits of `v` to a little-endian bit writer that flushes whole bytes.
struct ByteWriter {
  uint8_t* dst;
  uint64_t acc;
  int n;
  __device__ __forceinline__ void put(uint32_t v, int nbits) {
    acc |= (uint64_t)v << n;
    n += nbits;
    while (n >= 8) {
      *dst++ = (uint8_t)acc;
      acc >>= 8;
      n -= 8;
    }
  }
};

// 3-bit code fields are stored in groups of 32 codes, 12 bytes read as little-endian words
// W0, W1, W2.  Code j < 24 sits at bits 8 (j % 4) + 3 ((j % 8) / 4) of W_(j / 8); code 24 + r
// (r = 0..7) is bits 3 (r / 4) .. +2 of the 6-bit value T_k of byte lane k = r % 4, bit t of T_k
// being bit 8k + 6 + (t % 2) of W_(t / 2).  Masking a word (or its shift by 3) with 0x07070707
// then yields four codes, one per byte: ready-made v_perm selectors.
__device__ __forceinline__ uint32_t group3_top(uint32_t w0, uint32_t w1, uint32_t w2) {
  return ((w0 >> 6) & 0x03030303u) | ((w1 >> 4) & 0x0C0C0C0Cu) | ((w2 >> 2) & 0x30303030u);
}
__device__ __forceinline__ uint32_t group3_code(uint32_t w0, uint32_t w1, uint32_t w2, int j) {
  if (j < 24) {
    const uint32_t w = j < 8 ? w0 : (j < 16 ? w1 : w2);
    return (w >> (8 * (j & 3) + 3 * ((j >> 2) & 1))) & 7u;
  }
  const int r = j - 24;
  return (group3_top(w0, w1, w2) >> (8 * (r & 3) + 3 * (r >> 2))) & 7u;
}
// Place code j of a group (j a compile-time constant after unrolling).
__device__ __forceinline__ void group3_put(uint32_t (&w)[3], int j, uint32_t code) {
  if (j < 24) {
    w[j >> 3] |= code << (8 * (j & 3) + 3 * ((j >> 2) & 1));
    return;
  }
  const int r = j - 24, k = r & 3;
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const int t = 3 * (r >> 2) + b;
    w[t >> 1] |= ((code >> b) & 1u) << (8 * k + 6 + (t & 1));
  }
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    hipDeviceProp_t p;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess)
      n = p.multiProcessorCount;
    if (n <= 0) n = 256;
  }
  return n;
}

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Kernels that take more than 64 KB of dynamic LDS declare it once per kernel.
template <typename K>
void allow_lds(K kernel, size_t bytes) {
  if (bytes > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

// =========================================================================================
// Compression.  TurboQuant page (de.news.hada.io/topic?id=27867), "Funktionsweise von
// TurboQuant": step 1 rotates the vector at random and applies a fixed per-coordinate
// quantizer; step 2 adds a 1-bit QJL sketch of the residual ("QJL: Eine 1-Bit-Methode ohne
// Overhead").  Per token-head: r = |k|, x = Pi k, z = x * (sqrt(d)/r) rounded to float32,
// c = #{j : z >= tau_j}, e = x - (r32/sqrt(d)) gamma[c], rho = |e|, bit_j = [(S e)_j >= 0];
// values: codes and r_v only.  All of x, e, S e are float64 (MFMA f64), so the integer
// decisions match a float64 evaluation up to summation order.
//
// Wave tile = 16 token-heads.  MFMA 16x16x4 f64: lane l supplies A[l%16][l/16] and
// B[l/16][l%16]; accumulator register r of lane l holds C[l/16 + 4r][l%16].  A = rows of Pi
// (or S), permuted on the host so that lane group g = l/16, register r of output tile ct
// holds coordinate (d/4) g + 4 ct + r; B = the token's input at contraction index
// (d/4) g + s for k-step s.  Hence each lane ends up with d/4 consecutive rotated
// coordinates of one token, and the residual needed as the B operand of the projection at
// k-step s is the lane's own register (tile s/4, register s%4).
// =========================================================================================
typedef double f64x4 __attribute__((ext_vector_type(4)));

struct CompressArgs {
  Consts c;
  const float* pi_m;
  const float* s_m;
  const void* k;
  const void* v;
  tq_dtype dt;
  int heads;
  int64_t n_tokens, seq_stride, tok_stride, head_stride;
  uint8_t* records;
  int64_t capacity, first_slot;
  int64_t tiles_per_bh, n_tiles;
  int s_in_lds;
  PolarTables polar;
  const float* pi_t;      // generic kernel: Pi transposed [d][d], S transposed [d][m]
  const float* s_t;
};

template <int D>
__device__ __forceinline__ void rotate_tile(const float* lds_pi, const float (&in)[D / 4], int lane,
                                            f64x4 (&acc)[D / 16]) {
  constexpr int Q = D / 4, CT = D / 16;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < Q; ++s) {
    const double b = (double)in[s];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const double a = (double)lds_pi[(ct * Q + s) * 64 + lane];
      acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[ct], 0, 0, 0);
    }
  }
}

// Epilogue for one rotated vector held as acc[ct][r] = x[(d/4) g + 4 ct + r] (lane group g):
// z, codes packed into the code field starting at `field`.  Returns via `acc` the residual
// e = x - a*gamma[c] when want_residual.  3-bit fields use the 32-code group layout; at
// d = 64 two lane groups (g, g ^ 1: lanes l and l ^ 16) share a group and combine it with a
// shuffle, so every lane must call this.
template <int D>
__device__ __forceinline__ void quantize_rotated(f64x4 (&acc)[D / 16], double zscale, double a,
                                                 const float* levels, const float* bounds, int bits,
                                                 uint8_t* field, int g, bool want_residual) {
  constexpr int CT = D / 16, Q = D / 4;
  uint32_t codes[CT][4];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float z = (float)(acc[ct][r] * zscale);
      const uint32_t code = quantize_code(z, bounds);
      codes[ct][r] = code;
      if (want_residual) acc[ct][r] = acc[ct][r] - a * (double)levels[code];
    }
  }
  if (bits == 3) {
    uint32_t w[3] = {0u, 0u, 0u};
    if (Q == 32) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) group3_put(w, 4 * ct + r, codes[ct][r]);
    } else {   // Q == 16: this lane group holds codes 16 (g & 1) .. + 15 of group g / 2
      uint32_t w1[3] = {0u, 0u, 0u};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          group3_put(w, 4 * ct + r, codes[ct][r]);
          group3_put(w1, 16 + 4 * ct + r, codes[ct][r]);
        }
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        w[i] = (g & 1) ? w1[i] : w[i];
        w[i] |= __shfl_xor(w[i], 16);
      }
    }
    if (Q == 32 || (g & 1) == 0) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(field + 12 * (Q == 32 ? g : g >> 1));
      dst[0] = w[0];
      dst[1] = w[1];
      dst[2] = w[2];
    }
  } else {
    ByteWriter w{field + (Q * g * bits) / 8, 0, 0};
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) w.put(codes[ct][r], bits);
  }
}

// -----------------------------------------------------------------------------------------
// Polar key codes (TurboQuant page, section "PolarQuant"): the rotated key's coordinate pairs
// become (radius, angle), radii are paired again up to one radius.  This lane group holds
// coordinates [Q g, Q g + Q) (Q = d/4): levels 1 .. log2 Q are a subtree inside the lane, the
// two top levels pair the lane groups (g, g^1) and ({0,1}, {2,3}) by shuffles.  Angles are
// float64 atan2 (0 for two zeros); code = #{j : angle >= bound_j} on the float32 grid.  Codes
// go to `codes` (one byte per angle at d - (d >> (l-1)) + node for level l, packed later);
// x becomes the residual x - r u, u rebuilt top-down from the float64 cos / sin of the grid.
// Every lane of the wave must call this (shuffles).
// -----------------------------------------------------------------------------------------
// float64 products, sums and differences each rounded on their own (never fused into a
// multiply-add), in the order the host reference evaluates them
__device__ __forceinline__ double mul64(double a, double b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ double add64(double a, double b) {
#pragma clang fp contract(off)
  return a + b;
}
__device__ __forceinline__ double sub64(double a, double b) {
#pragma clang fp contract(off)
  return a - b;
}

__device__ __forceinline__ double polar_angle(double a, double b) {
  return (a == 0.0 && b == 0.0) ? 0.0 : atan2(b, a);
}

__device__ __forceinline__ uint32_t polar_code(double ang, const float* bounds_row, int nb) {
  uint32_t c = 0;
  for (int j = 0; j < nb; ++j) c += ang >= (double)bounds_row[j] ? 1u : 0u;
  return c;
}

template <int D>
__device__ __forceinline__ void polar_encode(f64x4 (&x)[D / 16], double r32, const PolarTables& pt,
                                             int b1, int bh, uint8_t* codes, int g) {
  constexpr int Q = D / 4, LQ = D == 128 ? 5 : 4;
  const int nb1 = (1 << b1) - 1, nbh = (1 << bh) - 1;
  double v[Q];
#pragma unroll
  for (int i = 0; i < Q; ++i) v[i] = x[i / 4][i % 4];
  uint32_t cd[Q];   // codes of the lane's subtree: level l at Q - (Q >> (l-1)) + node
#pragma unroll
  for (int l = 1, cnt = Q, off = 0; l <= LQ; ++l) {
#pragma unroll
    for (int i = 0; i < cnt / 2; ++i) {
      const double a = v[2 * i], b = v[2 * i + 1];
      const uint32_t c = polar_code(polar_angle(a, b), pt.bounds + (l - 1) * 16, l == 1 ? nb1 : nbh);
      cd[off + i] = c;
      codes[D - (D >> (l - 1)) + (Q >> l) * g + i] = (uint8_t)c;
      v[i] = sqrt(a * a + b * b);
    }
    off += cnt / 2;
    cnt /= 2;
  }
  // the two levels above the lane: pairs of lane groups
  const double r0 = v[0];
  const double o1 = __shfl_xor(r0, 16);
  const double l1 = (g & 1) ? o1 : r0, h1 = (g & 1) ? r0 : o1;
  const uint32_t c1 = polar_code(polar_angle(l1, h1), pt.bounds + LQ * 16, nbh);
  if ((g & 1) == 0) codes[D - (D >> LQ) + (g >> 1)] = (uint8_t)c1;
  const double r1 = sqrt(l1 * l1 + h1 * h1);
  const double o2 = __shfl_xor(r1, 32);
  const double l2 = (g & 2) ? o2 : r1, h2 = (g & 2) ? r1 : o2;
  const uint32_t c2 = polar_code(polar_angle(l2, h2), pt.bounds + (LQ + 1) * 16, nbh);
  if (g == 0) codes[D - (D >> (LQ + 1))] = (uint8_t)c2;
  // unit vector of the grid angles, top-down
  const double* top = pt.cs64 + 2 * ((LQ + 1) * 16 + c2);
  const double* mid = pt.cs64 + 2 * (LQ * 16 + c1);
  double u[Q];
  u[0] = ((g & 2) ? top[1] : top[0]) * ((g & 1) ? mid[1] : mid[0]);
#pragma unroll
  for (int l = LQ, cnt = 1; l >= 1; --l) {
    const int off = Q - (Q >> (l - 1));
#pragma unroll
    for (int i = cnt - 1; i >= 0; --i) {
      const double* cs = pt.cs64 + 2 * ((l - 1) * 16 + cd[off + i]);
      const double ui = u[i];
      u[2 * i + 1] = ui * cs[1];
      u[2 * i] = ui * cs[0];
    }
    cnt *= 2;
  }
#pragma unroll
  for (int i = 0; i < Q; ++i) x[i / 4][i % 4] = x[i / 4][i % 4] - r32 * u[i];
}

// Packs one token's polar code bytes into the key field: the level-1 stream (b1 bits per code)
// then levels 2..L (bh bits, zero-padded to whole 32-bit words).  `part` of 4 lanes per token.
__device__ __forceinline__ void polar_pack(const uint8_t* codes, int d, int b1, int bh, int l1_bytes,
                                           int kbytes, uint8_t* rec, int part) {
  const int nw1 = l1_bytes / 4, nw = kbytes / 4, n_up = d / 2 - 1;
  for (int w = part; w < nw; w += 4) {
    const bool lvl1 = w < nw1;
    const int bits = lvl1 ? b1 : bh, per = 32 / bits;
    const int first = (lvl1 ? w : w - nw1) * per;
    uint32_t word = 0;
    for (int i = 0; i < per; ++i) {
      const int idx = first + i;
      if (lvl1 || idx < n_up) word |= (uint32_t)codes[(lvl1 ? 0 : d / 2) + idx] << (bits * i);
    }
    reinterpret_cast<uint32_t*>(rec)[w] = word;
  }
}

// 512 threads (two waves per SIMD, sharing Pi and S in LDS) for scalar codes, so one wave's
// matrix-core products overlap the other's loads and epilogue; 256 for polar codes, whose
// angle work needs more registers than two waves per SIMD allow
constexpr int compress_threads(bool polar) { return polar ? 256 : 512; }

template <int D, bool POLAR>
__global__ __launch_bounds__(compress_threads(POLAR)) void compress_kernel(CompressArgs A) {
  constexpr int Q = D / 4, CT = D / 16;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const Consts& c = A.c;
  float* lds_pi = reinterpret_cast<float*>(smem);
  float* lds_s = lds_pi + D * D;
  float* lds_tab = lds_s + (A.s_in_lds ? c.m * D : 0);   // 4 x 16 floats
  uint8_t* stage_all = reinterpret_cast<uint8_t*>(lds_tab + 4 * kMaxLevels);
  uint8_t* codes_all = stage_all + (size_t)(blockDim.x >> 6) * 16 * c.rec_bytes;   // polar: [wave][16][D]

  // constants to LDS
  {
    const uint4* src = reinterpret_cast<const uint4*>(A.pi_m);
    uint4* dst = reinterpret_cast<uint4*>(lds_pi);
    for (int i = threadIdx.x; i < D * D / 4; i += blockDim.x) dst[i] = src[i];
    if (A.s_in_lds) {
      const uint4* s2 = reinterpret_cast<const uint4*>(A.s_m);
      uint4* d2 = reinterpret_cast<uint4*>(lds_s);
      for (int i = threadIdx.x; i < c.m * D / 4; i += blockDim.x) d2[i] = s2[i];
    }
    if (threadIdx.x < kMaxLevels) {
      lds_tab[threadIdx.x] = c.key_levels[threadIdx.x];
      lds_tab[kMaxLevels + threadIdx.x] = c.key_bounds[threadIdx.x];
      lds_tab[2 * kMaxLevels + threadIdx.x] = c.val_levels[threadIdx.x];
      lds_tab[3 * kMaxLevels + threadIdx.x] = c.val_bounds[threadIdx.x];
    }
  }
  __syncthreads();
  const float* s_src = A.s_in_lds ? lds_s : A.s_m;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int tok = lane & 15, g = lane >> 4;
  uint8_t* stage = stage_all + (size_t)wave * 16 * c.rec_bytes;
  const int mtiles = c.m / 16;

  for (int64_t tile = (int64_t)blockIdx.x * nwaves + wave; tile < A.n_tiles;
       tile += (int64_t)gridDim.x * nwaves) {
    const int64_t bh = tile / A.tiles_per_bh;
    const int64_t t0 = (tile % A.tiles_per_bh) * 16;
    const int64_t b = bh / A.heads;
    const int h = (int)(bh % A.heads);
    const int64_t t = t0 + tok;
    const bool valid = t < A.n_tokens;
    const int64_t row = b * A.seq_stride + t * A.tok_stride + h * A.head_stride + (int64_t)Q * g;
    uint8_t* rec = stage + tok * c.rec_bytes;

    // ---------------- keys ----------------
    float in[Q];
    load_row<Q>(A.k, A.dt, row, valid, in);
    double n2 = 0.0;
#pragma unroll
    for (int s = 0; s < Q; ++s) n2 += (double)in[s] * (double)in[s];
    n2 += __shfl_xor(n2, 16);
    n2 += __shfl_xor(n2, 32);
    const double r = sqrt(n2);
    const float r32 = (float)r;
    f64x4 x[CT];
    rotate_tile<D>(lds_pi, in, lane, x);
    const double zs = r > 0.0 ? c.sqrt_d / r : 0.0;
    const double a = (double)r32 / c.sqrt_d;
    uint8_t* pcodes = codes_all + ((size_t)wave * 16 + tok) * D;
    if constexpr (POLAR)
      polar_encode<D>(x, (double)r32, A.polar, c.pb1, c.pbh, pcodes, g);
    else
      quantize_rotated<D>(x, zs, a, lds_tab, lds_tab + kMaxLevels, c.kb, rec, g, true);
    double e2 = 0.0;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) e2 += x[ct][rr] * x[ct][rr];
    e2 += __shfl_xor(e2, 16);
    e2 += __shfl_xor(e2, 32);
    const float rho32 = (float)sqrt(e2);

    // ---------------- QJL sketch of the residual ----------------
    for (int pass = 0; pass * 8 < mtiles; ++pass) {
      f64x4 p[8];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) p[ct] = f64x4{0.0, 0.0, 0.0, 0.0};
      const int nt = min(8, mtiles - pass * 8);
#pragma unroll
      for (int s = 0; s < Q; ++s) {
        const double bop = x[s / 4][s % 4];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          if (ct < nt) {
            const double aop = (double)s_src[((pass * 8 + ct) * Q + s) * 64 + lane];
            p[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(aop, bop, p[ct], 0, 0, 0);
          }
        }
      }
      // lane group g holds p_j for j = (m/4) g + 32 pass + 4 ct + rr
      ByteWriter w{rec + c.kbytes + (c.m / 4) * g / 8 + 4 * pass, 0, 0};
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
        if (ct < nt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) w.put(((float)p[ct][rr] >= 0.0f) ? 1u : 0u, 1);
    }

    // ---------------- values ----------------
    load_row<Q>(A.v, A.dt, row, valid, in);
    double v2 = 0.0;
#pragma unroll
    for (int s = 0; s < Q; ++s) v2 += (double)in[s] * (double)in[s];
    v2 += __shfl_xor(v2, 16);
    v2 += __shfl_xor(v2, 32);
    const double rv = sqrt(v2);
    rotate_tile<D>(lds_pi, in, lane, x);
    const double zsv = rv > 0.0 ? c.sqrt_d / rv : 0.0;
    quantize_rotated<D>(x, zsv, 0.0, lds_tab + 2 * kMaxLevels, lds_tab + 3 * kMaxLevels, c.vb,
                        rec + c.kbytes + c.sbytes, g, false);

    if (g == 0) {
      float* nrm = reinterpret_cast<float*>(rec + c.norm_off);
      nrm[0] = r32;
      nrm[1] = rho32;
      nrm[2] = (float)rv;
    } else if (g == 1) {
      for (int i = c.norm_off + 12; i < c.rec_bytes; ++i) rec[i] = 0;
    }
    if constexpr (POLAR) {
      wave_lds_sync();
      polar_pack(pcodes, D, c.pb1, c.pbh, c.l1_bytes, c.kbytes, rec, g);
    }
    wave_lds_sync();
    // copy the staged records (16 consecutive slots of one (b, h)) to global memory
    const int64_t nvalid = min((int64_t)16, A.n_tokens - t0);
    const int n16 = (int)(nvalid * c.rec_bytes / 16);
    uint4* gdst = reinterpret_cast<uint4*>(A.records + ((bh * A.capacity) + A.first_slot + t0) * c.rec_bytes);
    const uint4* lsrc = reinterpret_cast<const uint4*>(stage);
    for (int i = lane; i < n16; i += 64) gdst[i] = lsrc[i];
    wave_lds_sync();
  }
}

// -----------------------------------------------------------------------------------------
// Compression at a head_dim without a matrix-core layout (a multiple of 8 up to 256, e.g. 200):
// one wave per token-head, lane i owns coordinates i, i + 64, ...; the rotation, residual and
// QJL projection are float64 FMA loops over the transposed matrices (coalesced rows), with the
// same decisions as the matrix-core kernel: z rounded to float32 against the float32 bounds,
// bit = [(float)(S e) >= 0].  The record is assembled in LDS and copied out as words.
// -----------------------------------------------------------------------------------------
constexpr int kGenMaxD = 256;
constexpr int kGenRecWords = 80;   // >= (256 * 4 / 8 + 256 / 8 + 256 * 4 / 8 + 12 rounded to 16) / 4

// Code field from one code byte per coordinate: 3-bit groups of 32 codes (the v_perm layout),
// a plain bitstream for the trailing partial group and for the other widths.  dst is zeroed.
__device__ __forceinline__ void pack_code_field(const uint8_t* codes, int d, int bits, uint32_t* dst, int lane) {
  if (bits == 3) {
    const int ng = d / 32;
    for (int g = lane; g < ng; g += 64) {
      uint32_t w[3] = {0u, 0u, 0u};
      for (int j = 0; j < 32; ++j) group3_put(w, j, codes[32 * g + j]);
      dst[3 * g] = w[0];
      dst[3 * g + 1] = w[1];
      dst[3 * g + 2] = w[2];
    }
    if (lane == 0) {
      for (int i = 32 * ng; i < d; ++i) {
        const int pos = 96 * ng + 3 * (i - 32 * ng);
        for (int t = 0; t < 3; ++t)
          dst[(pos + t) >> 5] |= (((uint32_t)codes[i] >> t) & 1u) << ((pos + t) & 31);
      }
    }
  } else {
    const int per = 32 / bits, nw = (d * bits + 31) / 32;
    for (int w = lane; w < nw; w += 64) {
      uint32_t word = 0u;
      for (int i = 0; i < per; ++i) {
        const int idx = w * per + i;
        if (idx < d) word |= (uint32_t)codes[idx] << (bits * i);
      }
      dst[w] = word;
    }
  }
}

// A wave compresses kGenTok consecutive tokens of one (sequence, head) together: every Pi^T or
// S^T entry it loads feeds one FMA per token, and the tokens' inputs sit side by side in LDS
// ([coordinate][token]), so one 16- or 32-byte LDS read serves all of them.
constexpr int kGenTok = 4;

__global__ __launch_bounds__(256) void compress_generic_kernel(CompressArgs A) {
  const Consts& c = A.c;
  __shared__ __attribute__((aligned(16))) double vin[4][kGenMaxD][kGenTok];
  __shared__ uint8_t cb[4][kGenTok][kGenMaxD];
  __shared__ uint32_t rw[4][kGenTok][kGenRecWords];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d = c.d, m = c.m, nrw = c.rec_bytes / 4;
  const int64_t tiles_per_bh = (A.n_tokens + kGenTok - 1) / kGenTok;
  for (int64_t item = (int64_t)blockIdx.x * 4 + wave; item < A.n_tiles; item += (int64_t)gridDim.x * 4) {
    const int64_t bh = item / tiles_per_bh, t0 = (item % tiles_per_bh) * kGenTok;
    const int64_t b = bh / A.heads;
    const int h = (int)(bh % A.heads);
    const int ntok = (int)min((int64_t)kGenTok, A.n_tokens - t0);
    for (int w = lane; w < kGenTok * nrw; w += 64) rw[wave][w / nrw][w % nrw] = 0u;
    float norms[kGenTok][3];
    for (int pass = 0; pass < 2; ++pass) {
      const void* src = pass == 0 ? A.k : A.v;
      for (int e = lane; e < kGenTok * d; e += 64) {
        const int tt = e / d, i = e % d;
        const int64_t row = b * A.seq_stride + (t0 + tt) * A.tok_stride + h * A.head_stride;
        vin[wave][i][tt] = tt < ntok ? (double)load_elem(src, A.dt, row + i) : 0.0;
      }
      wave_lds_sync();
      double zs[kGenTok], a[kGenTok];
      float r32[kGenTok];
#pragma unroll
      for (int tt = 0; tt < kGenTok; ++tt) {
        double n2 = 0.0;
        for (int i = lane; i < d; i += 64) n2 += vin[wave][i][tt] * vin[wave][i][tt];
        for (int o = 32; o >= 1; o >>= 1) n2 += __shfl_xor(n2, o);
        const double r = sqrt(n2);
        r32[tt] = (float)r;
        zs[tt] = r > 0.0 ? c.sqrt_d / r : 0.0;
        a[tt] = (double)r32[tt] / c.sqrt_d;
      }
      const float* bounds = pass == 0 ? c.key_bounds : c.val_bounds;
      const float* levels = pass == 0 ? c.key_levels : c.val_levels;
      double e[kGenMaxD / 64][kGenTok];
#pragma unroll
      for (int j = 0; j < kGenMaxD / 64; ++j) {
        const int i = lane + 64 * j;
#pragma unroll
        for (int tt = 0; tt < kGenTok; ++tt) e[j][tt] = 0.0;
        if (i < d) {
          double x[kGenTok] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
          for (int jj = 0; jj < d; ++jj) {
            const double p = (double)A.pi_t[(size_t)jj * d + i];
            const double4 v = *reinterpret_cast<const double4*>(&vin[wave][jj][0]);
            x[0] = fma(p, v.x, x[0]);
            x[1] = fma(p, v.y, x[1]);
            x[2] = fma(p, v.z, x[2]);
            x[3] = fma(p, v.w, x[3]);
          }
#pragma unroll
          for (int tt = 0; tt < kGenTok; ++tt) {
            const uint32_t code = quantize_code((float)(x[tt] * zs[tt]), bounds);
            cb[wave][tt][i] = (uint8_t)code;
            e[j][tt] = x[tt] - a[tt] * (double)levels[code];
          }
        }
      }
      wave_lds_sync();   // every lane is done reading vin and has written its codes
      const int fofs = pass == 0 ? 0 : (c.kbytes + c.sbytes) / 4;
      for (int tt = 0; tt < kGenTok; ++tt) {
        pack_code_field(cb[wave][tt], d, pass == 0 ? c.kb : c.vb, rw[wave][tt] + fofs, lane);
        norms[tt][pass == 0 ? 0 : 2] = r32[tt];
      }
      if (pass == 0) {
#pragma unroll
        for (int tt = 0; tt < kGenTok; ++tt) {
          double e2 = 0.0;
#pragma unroll
          for (int j = 0; j < kGenMaxD / 64; ++j) {
            const int i = lane + 64 * j;
            if (i < d) {
              vin[wave][i][tt] = e[j][tt];
              e2 += e[j][tt] * e[j][tt];
            }
          }
          for (int o = 32; o >= 1; o >>= 1) e2 += __shfl_xor(e2, o);
          norms[tt][1] = (float)sqrt(e2);
        }
        wave_lds_sync();
        for (int k0 = 0; k0 < m; k0 += 64) {
          const int k = k0 + lane;
          double p[kGenTok] = {0.0, 0.0, 0.0, 0.0};
          if (k < m) {
#pragma unroll 4
            for (int i = 0; i < d; ++i) {
              const double sv = (double)A.s_t[(size_t)i * m + k];
              const double4 v = *reinterpret_cast<const double4*>(&vin[wave][i][0]);
              p[0] = fma(sv, v.x, p[0]);
              p[1] = fma(sv, v.y, p[1]);
              p[2] = fma(sv, v.z, p[2]);
              p[3] = fma(sv, v.w, p[3]);
            }
          }
#pragma unroll
          for (int tt = 0; tt < kGenTok; ++tt) {
            const uint64_t bal = __ballot(k < m && (float)p[tt] >= 0.0f);
            if (lane == 0) {
              rw[wave][tt][c.kbytes / 4 + k0 / 32] = (uint32_t)bal;
              if (k0 + 32 < m) rw[wave][tt][c.kbytes / 4 + k0 / 32 + 1] = (uint32_t)(bal >> 32);
            }
          }
        }
      }
      wave_lds_sync();   // vin is reloaded by the next pass
    }
#pragma unroll
    for (int tt = 0; tt < kGenTok; ++tt)
#pragma unroll
      for (int f = 0; f < 3; ++f)
        if (lane == 3 * tt + f) rw[wave][tt][c.norm_off / 4 + f] = __float_as_uint(norms[tt][f]);
    wave_lds_sync();
    for (int e2 = lane; e2 < ntok * nrw; e2 += 64) {
      const int tt = e2 / nrw, w = e2 % nrw;
      uint32_t* dst = reinterpret_cast<uint32_t*>(A.records + (bh * A.capacity + A.first_slot + t0 + tt) * c.rec_bytes);
      dst[w] = rw[wave][tt][w];
    }
    wave_lds_sync();   // rw is cleared for the next item
  }
}

hipError_t launch_compress(const Consts& c, const DevConsts& dc, const void* k, const void* v,
                           tq_dtype dt, int batch, int64_t n_tokens, int heads, int64_t seq_stride,
                           int64_t tok_stride, int64_t head_stride, void* records,
                           int64_t capacity, int64_t first_slot, hipStream_t stream,
                           const ProfileEvents& ev) {
  CompressArgs A;
  A.c = c;
  A.pi_m = dc.pi_mfma;
  A.s_m = dc.s_mfma;
  A.k = k;
  A.v = v;
  A.dt = dt;
  A.heads = heads;
  A.n_tokens = n_tokens;
  A.seq_stride = seq_stride;
  A.tok_stride = tok_stride;
  A.head_stride = head_stride;
  A.records = static_cast<uint8_t*>(records);
  A.capacity = capacity;
  A.first_slot = first_slot;
  A.tiles_per_bh = (n_tokens + 15) / 16;
  A.n_tiles = A.tiles_per_bh * batch * heads;
  A.polar = dc.polar;
  A.pi_t = dc.pi_t;
  A.s_t = dc.s_t;
  if (c.d != 64 && c.d != 128) {
    A.n_tiles = (int64_t)batch * heads * ((n_tokens + kGenTok - 1) / kGenTok);   // one wave per kGenTok tokens
    const int64_t blocks = std::min<int64_t>((A.n_tiles + 3) / 4, (int64_t)num_cus() * 8);
    ev.before(stream);
    if (blocks > 0)
      hipLaunchKernelGGL(compress_generic_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, A);
    ev.after(stream);
    return hipGetLastError();
  }
  const int threads = compress_threads(c.polar != 0), nwaves = threads / 64;
  const size_t base = (size_t)c.d * c.d * 4 + 4 * kMaxLevels * 4 + (size_t)nwaves * 16 * c.rec_bytes +
                      (c.polar ? (size_t)nwaves * 16 * c.d : 0);
  const size_t with_s = base + (size_t)c.m * c.d * 4;
  A.s_in_lds = with_s <= 160 * 1024 ? 1 : 0;
  const size_t lds = A.s_in_lds ? with_s : base;
  int64_t blocks = (A.n_tiles + nwaves - 1) / nwaves;
  blocks = std::min<int64_t>(blocks, (int64_t)num_cus());
  ev.before(stream);
#define TQ_COMPRESS(D_, P_)                                                                      \
  {                                                                                              \
    allow_lds(compress_kernel<D_, P_>, lds);                                                     \
    hipLaunchKernelGGL((compress_kernel<D_, P_>), dim3((unsigned)blocks), dim3(threads), lds, stream, A); \
  }
  if (c.d == 128 && c.polar) TQ_COMPRESS(128, true)
  else if (c.d == 128) TQ_COMPRESS(128, false)
  else if (c.polar) TQ_COMPRESS(64, true)
  else TQ_COMPRESS(64, false)
#undef TQ_COMPRESS
  ev.after(stream);
  return hipGetLastError();
}

// Records from given float32 rotated inputs (the quantize + pack stage alone).
__global__ void debug_quantize_kernel(Consts c, const float* z_k, const float* p, const float* r_k,
                                      const float* rho, const float* z_v, const float* r_v,
                                      int64_t n, uint8_t* records) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  uint8_t* rec = records + t * c.rec_bytes;
  // a field of d codes: 3-bit codes in whole 32-code groups, then (d % 32 codes, head_dim 200)
  // a plain bitstream; every other width a plain bitstream; zero bytes up to the field's size
  auto put_codes = [&](uint8_t* field, const float* z, const float* bounds, int bits, int fbytes) {
    int i0 = 0;
    uint8_t* tail = field;
    if (bits == 3) {
      for (int gi = 0; gi < c.d / 32; ++gi) {
        uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 32; ++j) group3_put(w, j, quantize_code(z[32 * gi + j], bounds));
        uint32_t* dst = reinterpret_cast<uint32_t*>(field + 12 * gi);
        dst[0] = w[0];
        dst[1] = w[1];
        dst[2] = w[2];
      }
      i0 = c.d / 32 * 32;
      tail = field + 12 * (c.d / 32);
    }
    ByteWriter w{tail, 0, 0};
    for (int i = i0; i < c.d; ++i) w.put(quantize_code(z[i], bounds), bits);
    uint8_t* e = w.dst;
    if (w.n > 0) *e++ = (uint8_t)w.acc;
    while (e < field + fbytes) *e++ = 0;
  };
  put_codes(rec, z_k + t * c.d, c.key_bounds, c.kb, c.kbytes);
  ByteWriter ws{rec + c.kbytes, 0, 0};
  for (int j = 0; j < c.m; ++j) ws.put(p[t * c.m + j] >= 0.0f ? 1u : 0u, 1);
  put_codes(rec + c.kbytes + c.sbytes, z_v + t * c.d, c.val_bounds, c.vb, c.vbytes);
  float* nrm = reinterpret_cast<float*>(rec + c.norm_off);
  nrm[0] = r_k[t];
  nrm[1] = rho[t];
  nrm[2] = r_v[t];
  for (int i = c.norm_off + 12; i < c.rec_bytes; ++i) rec[i] = 0;
}

hipError_t launch_debug_quantize(const Consts& c, const float* z_k, const float* p, const float* r_k,
                                 const float* rho, const float* z_v, const float* r_v, int64_t n,
                                 void* records, hipStream_t stream) {
  const int threads = 128;
  hipLaunchKernelGGL(debug_quantize_kernel, dim3((unsigned)((n + threads - 1) / threads)), dim3(threads),
                     0, stream, c, z_k, p, r_k, rho, z_v, r_v, n, static_cast<uint8_t*>(records));
  return hipGetLastError();
}

// =========================================================================================
// Decode attention.  Query prep: q_x = Pi q, q_s = S q_x in float64 (one block of 256 threads
// per query).
// =========================================================================================
// y_i = sum_j M[i][j] v_j for i < rows (M float32 row-major [rows][d], v float64 in LDS, d a
// multiple of 4), by a block of 256 threads: output i of a pass of 32 rows is summed by eight
// adjacent lanes, lane ks taking columns 32 jj + 4 ks .. + 3, so that the eight read whole
// 128-byte lines of the row; the partial sums are combined by shuffles and lane ks = 0 calls
// out(i, y_i).
template <typename F>
__device__ __forceinline__ void block_gemv_f64(const float* __restrict__ M, const double* v, int rows, int d,
                                               F&& out) {
  // blockDim.x / 8 rows per pass: each pass is one memory round trip
  const int ks = threadIdx.x & 7, r0 = threadIdx.x >> 3, rpp = (int)blockDim.x >> 3;
  for (int i0 = 0; i0 < rows; i0 += rpp) {
    const int i = i0 + r0;
    double acc = 0.0;
    if (i < rows) {
#pragma unroll 4
      for (int c = 4 * ks; c < d; c += 32) {
        const float4 w = *reinterpret_cast<const float4*>(M + (int64_t)i * d + c);
        acc = fma((double)w.x, v[c], acc);
        acc = fma((double)w.y, v[c + 1], acc);
        acc = fma((double)w.z, v[c + 2], acc);
        acc = fma((double)w.w, v[c + 3], acc);
      }
    }
#pragma unroll
    for (int msk = 1; msk < 8; msk <<= 1) acc += __shfl_xor(acc, msk);
    if (ks == 0 && i < rows) out(i, acc);
  }
}

constexpr int kQueryPrepThreads = 1024;   // 128 rows of Pi or S per memory round trip
__device__ __forceinline__ void query_prep_block(const float* __restrict__ pi, const float* __restrict__ s, int d,
                                                 int m, const void* q, tq_dtype q_dt, float* qx_out,
                                                 float* qs_out, int64_t row) {
  __shared__ double qv[256];
  __shared__ double xv[256];
  for (int i = threadIdx.x; i < d; i += blockDim.x) qv[i] = (double)load_elem(q, q_dt, row * d + i);
  __syncthreads();
  block_gemv_f64(pi, qv, d, d, [&](int i, double y) {
    xv[i] = y;
    qx_out[row * d + i] = (float)y;
  });
  __syncthreads();
  block_gemv_f64(s, xv, m, d, [&](int k, double y) { qs_out[row * m + k] = (float)y; });
}

__global__ __launch_bounds__(kQueryPrepThreads) void query_prep_kernel(const float* __restrict__ pi,
                                                                       const float* __restrict__ s, int d, int m,
                                                                       const void* q, tq_dtype q_dt,
                                                                       float* qx_out, float* qs_out) {
  query_prep_block(pi, s, d, m, q, q_dt, qx_out, qs_out, blockIdx.x);   // row = flattened (b, h)
}

// -----------------------------------------------------------------------------------------
// Decode scan.  For the G query heads of one (sequence, KV head) and one chunk of tokens:
//   s_t = (r_k/sqrt(d)) sum_i q_x,i gamma_k[c_t,i] + sqrt(pi/2)/m rho_t sum_j q_s,j (2 bit_t,j - 1)
// (TurboQuant page, "QJL": the asymmetric estimator, full-precision query against 1-bit
// data), logit = scale * s_t, running softmax, o_x += p_t (r_v,t/sqrt(d)) gamma_v[c^v_t].
// Key sums are LUT-GEMV lookups (as the Self-Indexing page, "Methodologie" 3, does for its
// selector): a table of sum_{i in pair} q_x,i gamma[c_i] for every pair of codes, and a table
// of sum_{j in byte} q_s,j (+-1) for every byte of sign bits, both in LDS, each entry holding
// the HPL heads of one head group.
// Lane layout: LPT = (d/32) * (G/HPL) lanes per token; lane (cq, hg) handles coordinates
// [32 cq, 32 cq + 32) and heads [HPL hg, HPL hg + HPL).  Lanes keep private running maxima
// (raised lazily, only when a logit exceeds the max by kLazy) and private accumulators that
// are merged across lanes and waves at the end of the chunk.
// -----------------------------------------------------------------------------------------
constexpr float kLazy = 8.0f;
constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
constexpr int kDecodeThreads = 512;

struct DecodeArgs {
  const float* qx;
  const float* qs;
  const uint32_t* bop;    // matrix-core kernel: per-lane query operands (mfma_prep_kernel)
  const uint8_t* records;
  const int32_t* seq_lens;
  const int32_t* sel_idx;
  const int32_t* gate;    // [B][Hq] nonzero: the head reads the cold tokens (NULL: all do)
  float* part;
  float* logits;
  int64_t capacity, logit_stride;
  int d, m, kbytes, sbytes, rec_bytes, norm_off;
  int kb, vb;             // code widths (the generic-head_dim kernel reads them at run time)
  int G, q_heads, kv_heads, k_sel, chunk, n_chunks, sign_bytes;
  float scale, inv_sqrt_d, qjl_coef, key_fix;
  float key_levels[kMaxLevels];
  float val_levels[kMaxLevels];
  // polar key codes
  const float* pcs;       // cos / sin of the float32 angle grids, [8][16][2]
  int pb1, pbh, plevels, l1_bytes;
};

template <int NW>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[NW], int pos, int nbits) {
  const int wi = pos >> 5, sh = pos & 31;
  uint32_t v = w[wi] >> sh;
  if (sh + nbits > 32 && wi + 1 < NW) v |= w[wi + 1] << (32 - sh);
  return v & ((1u << nbits) - 1u);
}

template <int HPL, int BK, int BV, bool POLAR = false>
__global__ __launch_bounds__(kDecodeThreads) void decode_scan_kernel(DecodeArgs A) {
  constexpr bool kPairs = BK <= 3 && !POLAR;
  constexpr int kEnt = kPairs ? (1 << (2 * BK)) : (1 << BK);   // entries per key table
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int d = A.d, G = A.G, NHG = G / HPL, LPTc = d / 32, LPT = LPTc * NHG, TPW = 64 / LPT;
  const int b = blockIdx.z, hkv = blockIdx.y, chunk = blockIdx.x;
  // polar: one table per level-1 pair, 16 entries (q_2p cos + q_2p+1 sin of each grid angle),
  // then the cos / sin of the grids of levels 2..L
  const int nkt = (kPairs || POLAR) ? d / 2 : d;               // key tables per head group
  const int sgrp = A.sign_bytes ? A.m / 8 : A.m / 4;            // sign tables per head group
  const int sent = A.sign_bytes ? 256 : 16;
  float* lut_k = lds;                                           // [NHG][nkt][kEnt][HPL]
  float* lut_s = lut_k + NHG * nkt * kEnt * HPL;                // [NHG][sgrp][sent][HPL]
  float* gam_v = lut_s + NHG * sgrp * sent * HPL;               // [16]
  float* pcs_up = gam_v + kMaxLevels;                            // polar: [L-1][16][2]

  const int64_t qrow0 = ((int64_t)b * A.q_heads + (int64_t)hkv * G);  // first query head row
  if (A.gate) {            // no head of the group reads the cold tokens: the merge ignores them
    bool any = false;
    for (int j = 0; j < G; ++j) any = any || A.gate[qrow0 + j] != 0;
    if (!any) return;
  }
  // ---- LUT build: one thread per table row (head group, table, head), whose one or two query
  // coordinates are loaded once; the row's entries are then written from registers ----
  {
    const float* qx = A.qx + qrow0 * d;
    const int nrow_k = NHG * nkt * HPL;
    for (int r = threadIdx.x; r < nrow_k; r += blockDim.x) {
      const int j = r % HPL, tbl = (r / HPL) % nkt, hg = r / HPL / nkt;
      const float* qh = qx + (int64_t)(hg * HPL + j) * d;
      float* dst = lut_k + (int64_t)(hg * nkt + tbl) * kEnt * HPL + j;
      if (POLAR) {
        const float q0 = qh[2 * tbl], q1 = qh[2 * tbl + 1];
#pragma unroll
        for (int ent = 0; ent < kEnt; ++ent)
          dst[ent * HPL] = fmaf(q1, A.pcs[2 * ent + 1], q0 * A.pcs[2 * ent]);
      } else if (kPairs) {
        // pair p of a 32-coordinate group: 2-bit codes (2p, 2p+1), adjacent in the bitstream;
        // 3-bit codes (8 (p / 4) + p % 4, that + 4), one 6-bit byte field of the group layout
        const int pp = tbl & 15, g32 = 32 * (tbl >> 4);
        const int i0 = BK == 3 ? g32 + 8 * (pp >> 2) + (pp & 3) : 2 * tbl;
        const int i1 = BK == 3 ? i0 + 4 : 2 * tbl + 1;
        const float q0 = qh[i0], q1 = qh[i1];
#pragma unroll
        for (int ent = 0; ent < kEnt; ++ent) {
          const int c0 = ent & ((1 << BK) - 1), c1 = ent >> BK;
          dst[ent * HPL] = fmaf(q1, A.key_levels[c1], q0 * A.key_levels[c0]);
        }
      } else {
        const float q0 = qh[tbl];
#pragma unroll
        for (int ent = 0; ent < kEnt; ++ent) dst[ent * HPL] = q0 * A.key_levels[ent];
      }
    }
    // sign tables: one thread per (head group, table, head, 16 consecutive entries)
    const float* qs = A.qs + qrow0 * A.m;
    const int per = A.sign_bytes ? 8 : 4;
    const int nsub = sent / 16;
    const int nrow_s = NHG * sgrp * HPL * nsub;
    for (int r = threadIdx.x; r < nrow_s; r += blockDim.x) {
      const int sub = r % nsub, j = (r / nsub) % HPL, grp = (r / nsub / HPL) % sgrp, hg = r / nsub / HPL / sgrp;
      const float* qh = qs + (int64_t)(hg * HPL + j) * A.m + grp * per;
      float qv8[8];
#pragma unroll
      for (int kq = 0; kq < 8; ++kq) {
        qv8[kq] = 0.0f;
        if (kq < per) qv8[kq] = qh[kq];
      }
      float* dst = lut_s + ((int64_t)(hg * sgrp + grp) * sent + 16 * sub) * HPL + j;
#pragma unroll
      for (int e16 = 0; e16 < 16; ++e16) {
        const int ent = 16 * sub + e16;
        float val = 0.0f;
#pragma unroll
        for (int kq = 0; kq < 8; ++kq)
          if (kq < per) val += ((ent >> kq) & 1) ? qv8[kq] : -qv8[kq];
        dst[e16 * HPL] = val;
      }
    }
    if (threadIdx.x < kMaxLevels) gam_v[threadIdx.x] = A.val_levels[threadIdx.x];
    if (POLAR)
      for (int i = threadIdx.x; i < (A.plevels - 1) * 32; i += blockDim.x) pcs_up[i] = A.pcs[32 + i];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int lt = lane % LPT, cq = lt % LPTc, hg = lt / LPTc, slot = lane / LPT;
  // polar: this lane's 32 coordinates are the subtree of level-5 node cq.  Byte offset of the
  // 32-bit word holding each level's codes for it (levels 2..5: 32 >> l consecutive codes;
  // levels 6..L: the one ancestor), and the bit shift of the first code in that word.
  int pw[kMaxPolarLevels], psh[kMaxPolarLevels];
  if (POLAR) {
#pragma unroll
    for (int l = 2; l < kMaxPolarLevels + 1; ++l) {
      if (l > A.plevels) break;
      const int lev_off = (d / 2 - (d >> (l - 1))) * A.pbh;                  // level start (bits)
      const int node = l <= 5 ? cq * (32 >> l) : cq >> (l - 5);
      const int bit = lev_off + node * A.pbh;
      pw[l - 2] = A.l1_bytes + 4 * (bit >> 5);
      psh[l - 2] = bit & 31;
    }
  }
  const bool gather = A.sel_idx != nullptr;
  int n = gather ? A.k_sel : min((int64_t)A.seq_lens[b], A.capacity);
  const int c0 = chunk * A.chunk, c1 = min(n, c0 + A.chunk);
  const uint8_t* recs = A.records + ((int64_t)b * A.kv_heads + hkv) * A.capacity * A.rec_bytes;
  const int32_t* sel = gather ? A.sel_idx + ((int64_t)b * A.kv_heads + hkv) * A.k_sel : nullptr;

  float mrun[HPL], lsum[HPL], acc[HPL][32];
#pragma unroll
  for (int j = 0; j < HPL; ++j) {
    mrun[j] = kNegInf;
    lsum[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[j][i] = 0.0f;
  }
  const float* lk = lut_k + (hg * nkt + (kPairs ? 16 : 32) * cq) * kEnt * HPL;
  const int nsw = A.m / 32;   // sign dwords per token

  for (int base = c0 + wave * TPW; base < c1; base += nwaves * TPW) {
    const int pos = base + slot;
    int64_t t = pos;
    bool valid = pos < c1;
    if (gather && valid) t = sel[pos];
    valid = valid && t >= 0 && t < A.capacity;
    const uint8_t* rec = recs + (valid ? t : 0) * A.rec_bytes;
    uint32_t kw[BK], vw[BV];
#pragma unroll
    for (int i = 0; i < BK; ++i)
      kw[i] = (valid && !POLAR) ? reinterpret_cast<const uint32_t*>(rec + cq * 4 * BK)[i] : 0u;
#pragma unroll
    for (int i = 0; i < BV; ++i)
      vw[i] = valid ? reinterpret_cast<const uint32_t*>(rec + A.kbytes + A.sbytes + cq * 4 * BV)[i] : 0u;
    const float* nrm = reinterpret_cast<const float*>(rec + A.norm_off);
    const float rk = valid ? nrm[0] : 0.0f, rho = valid ? nrm[1] : 0.0f, rv = valid ? nrm[2] : 0.0f;

    // key code part: sum over this lane's 32 coordinates
    float cs[HPL];
#pragma unroll
    for (int j = 0; j < HPL; ++j) cs[j] = 0.0f;
    if (POLAR) {
      // level-1 codes: 16 codes of b1 bits from byte 2 b1 cq
      const int b1 = A.pb1, bh = A.pbh;
      const uint32_t* l1w = reinterpret_cast<const uint32_t*>(rec + 2 * b1 * cq);
      const uint32_t w0 = valid ? l1w[0] : 0u;
      const uint32_t w1 = (valid && b1 == 4) ? l1w[1] : 0u;
      uint32_t uw[kMaxPolarLevels];
#pragma unroll
      for (int l = 2; l <= kMaxPolarLevels; ++l)
        uw[l - 2] = (valid && l <= A.plevels) ? *reinterpret_cast<const uint32_t*>(rec + pw[l - 2]) >> psh[l - 2] : 0u;
      // scale of the lane's subtree root: cos or sin of each ancestor's angle
      float sroot = 1.0f;
#pragma unroll
      for (int l = 6; l <= kMaxPolarLevels; ++l) {
        if (l <= A.plevels) {
          const uint32_t c = uw[l - 2] & ((1u << bh) - 1u);
          const float2 t = reinterpret_cast<const float2*>(pcs_up)[(l - 2) * 16 + c];
          sroot *= ((cq >> (l - 6)) & 1) ? t.y : t.x;
        }
      }
      // levels 5..3 inside the lane: scales of the 8 level-2 nodes
      float sc[8];
      sc[0] = sroot;
#pragma unroll
      for (int l = 5, cnt = 1; l >= 3; --l, cnt *= 2) {
#pragma unroll
        for (int i = cnt - 1; i >= 0; --i) {
          const uint32_t c = (uw[l - 2] >> (bh * i)) & ((1u << bh) - 1u);
          const float2 t = reinterpret_cast<const float2*>(pcs_up)[(l - 2) * 16 + c];
          const float si = sc[i];
          sc[2 * i + 1] = si * t.y;
          sc[2 * i] = si * t.x;
        }
      }
      // level 2 (angle psi) over level-1 pairs (2k, 2k+1): sum_j q.(s cos psi T1[2k] + s sin psi T1[2k+1])
      const float* lkp = lut_k + (hg * nkt + 16 * cq) * kEnt * HPL;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t c2 = (uw[0] >> (bh * k)) & ((1u << bh) - 1u);
        const float2 t = reinterpret_cast<const float2*>(pcs_up)[c2];
        const float a = sc[k] * t.x, bb = sc[k] * t.y;
        const int ia = 2 * k, ib = 2 * k + 1;
        const uint32_t ca = ((b1 == 4 && ia >= 8) ? w1 : w0) >> ((b1 * ia) & 31) & ((1u << b1) - 1u);
        const uint32_t cb = ((b1 == 4 && ib >= 8) ? w1 : w0) >> ((b1 * ib) & 31) & ((1u << b1) - 1u);
        const float* ea = lkp + (ia * kEnt + ca) * HPL;
        const float* eb = lkp + (ib * kEnt + cb) * HPL;
        if (HPL == 4) {
          const float4 va = *reinterpret_cast<const float4*>(ea);
          const float4 vb = *reinterpret_cast<const float4*>(eb);
          cs[0] = fmaf(bb, vb.x, fmaf(a, va.x, cs[0]));
          cs[HPL > 1 ? 1 : 0] = fmaf(bb, vb.y, fmaf(a, va.y, cs[HPL > 1 ? 1 : 0]));
          cs[HPL > 2 ? 2 : 0] = fmaf(bb, vb.z, fmaf(a, va.z, cs[HPL > 2 ? 2 : 0]));
          cs[HPL > 3 ? 3 : 0] = fmaf(bb, vb.w, fmaf(a, va.w, cs[HPL > 3 ? 3 : 0]));
        } else {
#pragma unroll
          for (int j = 0; j < HPL; ++j) cs[j] = fmaf(bb, eb[j], fmaf(a, ea[j], cs[j]));
        }
      }
    } else if (kPairs) {
      const uint32_t top = BK == 3 ? group3_top(kw[0], kw[BK > 1 ? 1 : 0], kw[BK > 2 ? 2 : 0]) : 0u;
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const uint32_t idx = BK == 3 ? ((p < 12 ? kw[(p >> 2) < BK ? (p >> 2) : 0] : top) >> (8 * (p & 3))) & 63u
                                     : field<BK>(kw, 2 * p * BK, 2 * BK);
        const float* e = lk + (p * kEnt + idx) * HPL;
        if (HPL == 4) {
          const float4 v = *reinterpret_cast<const float4*>(e);
          cs[0] += v.x; cs[HPL > 1 ? 1 : 0] += v.y; cs[HPL > 2 ? 2 : 0] += v.z; cs[HPL > 3 ? 3 : 0] += v.w;
        } else {
#pragma unroll
          for (int j = 0; j < HPL; ++j) cs[j] += e[j];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t idx = field<BK>(kw, i * BK, BK);
        const float* e = lk + (i * kEnt + idx) * HPL;
        if (HPL == 4) {
          const float4 v = *reinterpret_cast<const float4*>(e);
          cs[0] += v.x; cs[HPL > 1 ? 1 : 0] += v.y; cs[HPL > 2 ? 2 : 0] += v.z; cs[HPL > 3 ? 3 : 0] += v.w;
        } else {
#pragma unroll
          for (int j = 0; j < HPL; ++j) cs[j] += e[j];
        }
        // keep at most 8 table reads in flight (register pressure next to 4 x 32 accumulators)
        if (HPL == 4 && (i % 8) == 7) __builtin_amdgcn_sched_barrier(0);
      }
    }
    // QJL part: this lane's sign dwords
    float qsum[HPL];
#pragma unroll
    for (int j = 0; j < HPL; ++j) qsum[j] = 0.0f;
    for (int jw = cq; jw < nsw; jw += LPTc) {
      const uint32_t sw = valid ? reinterpret_cast<const uint32_t*>(rec + A.kbytes)[jw] : 0u;
      if (A.sign_bytes) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float* e = lut_s + ((hg * sgrp + jw * 4 + q4) * 256 + ((sw >> (8 * q4)) & 255u)) * HPL;
#pragma unroll
          for (int j = 0; j < HPL; ++j) qsum[j] += e[j];
        }
      } else {
#pragma unroll
        for (int q8 = 0; q8 < 8; ++q8) {
          const float* e = lut_s + ((hg * sgrp + jw * 8 + q8) * 16 + ((sw >> (4 * q8)) & 15u)) * HPL;
#pragma unroll
          for (int j = 0; j < HPL; ++j) qsum[j] += e[j];
        }
      }
    }
    float logit[HPL];
    const float ak = POLAR ? rk : rk * A.inv_sqrt_d, aq = A.qjl_coef * rho;
#pragma unroll
    for (int j = 0; j < HPL; ++j) {
      float sj = fmaf(aq, qsum[j], ak * cs[j]);
      for (int msk = 1; msk < LPTc; msk <<= 1) sj += __shfl_xor(sj, msk);
      logit[j] = A.scale * sj;
    }
    if (A.logits && valid && cq == 0) {
#pragma unroll
      for (int j = 0; j < HPL; ++j)
        A.logits[(qrow0 + hg * HPL + j) * A.logit_stride + pos] = logit[j];
    }
    // lazy online softmax
    float w[HPL];
#pragma unroll
    for (int j = 0; j < HPL; ++j) {
      if (valid && logit[j] > mrun[j] + kLazy) {
        const float f = mrun[j] == kNegInf ? 0.0f : __expf(mrun[j] - logit[j]);
        lsum[j] *= f;
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[j][i] *= f;
        mrun[j] = logit[j];
      }
      const float p = valid ? __expf(logit[j] - mrun[j]) : 0.0f;
      lsum[j] += p;
      w[j] = p * rv * A.inv_sqrt_d;
    }
    // values
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t vc = BV == 3 ? group3_code(vw[0], vw[BV > 1 ? 1 : 0], vw[BV > 2 ? 2 : 0], i)
                                  : field<BV>(vw, i * BV, BV);
      const float gv = gam_v[vc];
#pragma unroll
      for (int j = 0; j < HPL; ++j) acc[j][i] = fmaf(w[j], gv, acc[j][i]);
    }
  }

  // ---- combine the TPW token slots of each wave (butterfly over the slot bits of the lane),
  // then the waves of the block through LDS, one head at a time ----
  for (int o = LPT; o < 64; o <<= 1) {
#pragma unroll
    for (int j = 0; j < HPL; ++j) {
      const float mo = __shfl_xor(mrun[j], o), lo = __shfl_xor(lsum[j], o);
      const float mn = fmaxf(mrun[j], mo);
      const float f = mrun[j] == kNegInf ? 0.0f : __expf(mrun[j] - mn);
      const float fo = mo == kNegInf ? 0.0f : __expf(mo - mn);
      lsum[j] = fmaf(lsum[j], f, lo * fo);
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[j][i] = fmaf(acc[j][i], f, __shfl_xor(acc[j][i], o) * fo);
      mrun[j] = mn;
    }
  }
  __syncthreads();   // the LUTs are no longer needed
  const int nthr = blockDim.x;
  float* pacc = lds;                     // [nthr][33]  accumulators of head j (+1 pad)
  float* pf = pacc + nthr * 33;          // [nthr]      per-lane scale exp(m - M)
  float* pl = pf + nthr;                 // [nthr]      per-lane l
  float* pm = pl + nthr;                 // [NHG]       block maximum per head group
  const int stride = d + 2;
  for (int j = 0; j < HPL; ++j) {
#pragma unroll
    for (int i = 0; i < 32; ++i) pacc[threadIdx.x * 33 + i] = acc[j][i];
    pf[threadIdx.x] = mrun[j];
    pl[threadIdx.x] = lsum[j];
    __syncthreads();
    // block maximum of head (hg, j) over the waves (slot 0 of each wave holds its combined
    // partial; cq = 0 lanes carry m and l)
    for (int hh = threadIdx.x; hh < NHG; hh += nthr) {
      float mx = kNegInf;
      for (int t2 = hh * LPTc; t2 < nthr; t2 += 64) mx = fmaxf(mx, pf[t2]);
      pm[hh] = mx;
    }
    __syncthreads();
    {
      const int hh = (threadIdx.x % LPT) / LPTc;
      const float mt = pf[threadIdx.x], mx = pm[hh];
      const float f = mt == kNegInf ? 0.0f : __expf(mt - mx);
      __syncthreads();
      pf[threadIdx.x] = f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < NHG * stride; e += nthr) {
      const int hh = e / stride, col = e % stride;
      float v;
      if (col == 0) {
        v = pm[hh];
      } else if (col == 1) {
        v = 0.0f;
        for (int t2 = hh * LPTc; t2 < nthr; t2 += 64) v += pl[t2] * pf[t2];
      } else {
        const int i = col - 2, cqo = i / 32, io = i % 32;
        v = 0.0f;
        for (int t2 = hh * LPTc + cqo; t2 < nthr; t2 += 64) v += pacc[t2 * 33 + io] * pf[t2];
      }
      A.part[((qrow0 + hh * HPL + j) * A.n_chunks + chunk) * stride + col] = v;
    }
    __syncthreads();
  }
}

// -----------------------------------------------------------------------------------------
// Direct scan for short caches (up to a few thousand tokens per (sequence, KV head)): one
// workgroup per (chunk of at most 64 tokens, KV head, sequence).  The chunk's codes are
// unpacked into LDS, then every (token, head) estimate, the chunk's softmax and every (head,
// coordinate) output are computed directly from q_x, q_s and the level tables, with no
// per-query lookup tables, whose build would outweigh a few dozen tokens.  Same estimator and
// the same partial format (m, l, o_x) as decode_scan_kernel.
// -----------------------------------------------------------------------------------------
constexpr int kSmallThreads = 256;
constexpr int64_t kSmallMaxN = 4096;      // tokens per (sequence, KV head) for the direct kernel
constexpr int kSmallMaxTok = 64;
constexpr int kSmallMaxG = 16;
constexpr int kSmallMaxM = 128;

template <int D, int BK, int BV>
__global__ __launch_bounds__(kSmallThreads) void decode_small_kernel(DecodeArgs A) {
  constexpr int NG32 = D / 32;
  __shared__ float qx[kSmallMaxG][D + 1];
  __shared__ float qs[kSmallMaxG][kSmallMaxM + 1];
  __shared__ __attribute__((aligned(4))) uint8_t kc[kSmallMaxTok][D];          // key codes
  __shared__ __attribute__((aligned(4))) uint8_t vc[kSmallMaxTok][D];          // value codes
  __shared__ __attribute__((aligned(4))) uint8_t sb[kSmallMaxTok][kSmallMaxM]; // QJL bits
  __shared__ float nr[kSmallMaxTok][3];            // r_k, rho, r_v
  __shared__ int ok_t[kSmallMaxTok];
  __shared__ float lg[kSmallMaxG][kSmallMaxTok + 1];   // logits, then weights p r_v / sqrt(d)
  __shared__ float hm[kSmallMaxG], hl[kSmallMaxG];
  __shared__ float kl[kMaxLevels], vl[kMaxLevels];
  const int G = A.G, m = A.m, TOK = A.chunk, tid = threadIdx.x;
  const int b = blockIdx.z, hkv = blockIdx.y, chunk = blockIdx.x;
  const int64_t qrow0 = (int64_t)b * A.q_heads + (int64_t)hkv * G;
  if (A.gate) {            // no head of the group reads the cold tokens: the merge ignores them
    bool any = false;
    for (int j = 0; j < G; ++j) any = any || A.gate[qrow0 + j] != 0;
    if (!any) return;
  }
  const bool gather = A.sel_idx != nullptr;
  const int n = gather ? A.k_sel : (int)min((int64_t)A.seq_lens[b], A.capacity);
  const int c0 = chunk * TOK, nt = max(0, min(TOK, n - c0));
  const uint8_t* recs = A.records + ((int64_t)b * A.kv_heads + hkv) * A.capacity * A.rec_bytes;
  for (int e = tid; e < G * D; e += kSmallThreads) qx[e / D][e % D] = A.qx[(qrow0 + e / D) * D + e % D];
  for (int e = tid; e < G * m; e += kSmallThreads) qs[e / m][e % m] = A.qs[(qrow0 + e / m) * m + e % m];
  if (tid < kMaxLevels) {
    kl[tid] = A.key_levels[tid];
    vl[tid] = A.val_levels[tid];
  }
  // unpack: per token, NG32 key groups, NG32 value groups, m / 32 sign words and the norms
  const int nsw = m / 32, per_t = 2 * NG32 + nsw + 1;
  for (int e = tid; e < nt * per_t; e += kSmallThreads) {
    const int t = e / per_t, pt = e % per_t;
    int64_t tok = c0 + t;
    bool ok = true;
    if (gather) {
      tok = A.sel_idx[((int64_t)b * A.kv_heads + hkv) * A.k_sel + c0 + t];
      ok = tok >= 0 && tok < A.capacity;
    }
    const uint8_t* rec = recs + (ok ? tok : 0) * A.rec_bytes;
    if (pt < 2 * NG32) {
      const bool key = pt < NG32;
      const int g = key ? pt : pt - NG32;
      uint32_t w[4];
      const uint32_t* src = reinterpret_cast<const uint32_t*>(
          rec + (key ? g * 4 * BK : A.kbytes + A.sbytes + g * 4 * BV));
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = i < (key ? BK : BV) ? src[i] : 0u;
      uint32_t* dst = reinterpret_cast<uint32_t*>(key ? &kc[t][32 * g] : &vc[t][32 * g]);
      const int nb = key ? BK : BV;
#pragma unroll
      for (int j4 = 0; j4 < 8; ++j4) {          // four codes per word
        uint32_t word = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = 4 * j4 + u;
          const uint32_t code = nb == 3 ? group3_code(w[0], w[1], w[2], j) : field<4>(w, j * nb, nb);
          word |= code << (8 * u);
        }
        dst[j4] = word;
      }
    } else if (pt < 2 * NG32 + nsw) {
      const int wi = pt - 2 * NG32;
      const uint32_t sw = reinterpret_cast<const uint32_t*>(rec + A.kbytes)[wi];
      uint32_t* dst = reinterpret_cast<uint32_t*>(&sb[t][32 * wi]);
#pragma unroll
      for (int j4 = 0; j4 < 8; ++j4) {
        const uint32_t nib = (sw >> (4 * j4)) & 15u;   // bits 4 j4 .. 4 j4 + 3, one per byte
        dst[j4] = (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
      }
    } else {
      const float* f = reinterpret_cast<const float*>(rec + A.norm_off);
      nr[t][0] = f[0];
      nr[t][1] = f[1];
      nr[t][2] = f[2];
      ok_t[t] = ok ? 1 : 0;
    }
  }
  __syncthreads();
  // estimates: L adjacent lanes per (token, head), each over every L-th coordinate and bit
  const int items = nt * G;
  int L = 1;
  while (L < 8 && items * L * 2 <= kSmallThreads) L *= 2;
  for (int i0 = 0; i0 < items; i0 += kSmallThreads / L) {
    const int it = i0 + tid / L, s = tid % L;
    const int t = it / G, h = it % G;
    float dot = 0.0f, qd = 0.0f;
    if (it < items) {
      for (int i = s; i < D; i += L) dot = fmaf(qx[h][i], kl[kc[t][i]], dot);
      for (int j = s; j < m; j += L) qd += sb[t][j] ? qs[h][j] : -qs[h][j];
    }
    for (int msk = 1; msk < L; msk <<= 1) {
      dot += __shfl_xor(dot, msk);
      qd += __shfl_xor(qd, msk);
    }
    if (it < items && s == 0) {
      const float logit = ok_t[t] ? A.scale * fmaf(A.qjl_coef * nr[t][1], qd, nr[t][0] * A.inv_sqrt_d * dot)
                                  : kNegInf;
      lg[h][t] = logit;
      if (A.logits && ok_t[t]) A.logits[(qrow0 + h) * A.logit_stride + c0 + t] = logit;
    }
  }
  __syncthreads();
  // the chunk's softmax per head: m, l, and the value weights p r_v / sqrt(d)
  for (int h = tid; h < G; h += kSmallThreads) {
    float mx = kNegInf;
    for (int t = 0; t < nt; ++t) mx = fmaxf(mx, lg[h][t]);
    float l = 0.0f;
    for (int t = 0; t < nt; ++t) {
      const float p = (mx == kNegInf || lg[h][t] == kNegInf) ? 0.0f : __expf(lg[h][t] - mx);
      l += p;
      lg[h][t] = p * nr[t][2] * A.inv_sqrt_d;
    }
    hm[h] = mx;
    hl[h] = l;
  }
  __syncthreads();
  const int stride = D + 2;
  for (int e = tid; e < G * D; e += kSmallThreads) {
    const int h = e / D, i = e % D;
    float o = 0.0f;
    for (int t = 0; t < nt; ++t) o = fmaf(lg[h][t], vl[vc[t][i]], o);
    A.part[((qrow0 + h) * A.n_chunks + chunk) * stride + 2 + i] = o;
  }
  for (int h = tid; h < G; h += kSmallThreads) {
    A.part[((qrow0 + h) * A.n_chunks + chunk) * stride] = hm[h];
    A.part[((qrow0 + h) * A.n_chunks + chunk) * stride + 1] = hl[h];
  }
}

template <int D>
static void launch_small_d(const DecodeArgs& a, int kb, int vb, dim3 grid, hipStream_t st) {
#define TQ_SM(BK_, BV_)                                                                           \
  if (kb == BK_ && vb == BV_) {                                                                   \
    hipLaunchKernelGGL((decode_small_kernel<D, BK_, BV_>), grid, dim3(kSmallThreads), 0, st, a);  \
    return;                                                                                       \
  }
  TQ_SM(1, 1) TQ_SM(1, 2) TQ_SM(1, 3) TQ_SM(1, 4) TQ_SM(2, 1) TQ_SM(3, 1) TQ_SM(4, 1)
  TQ_SM(2, 2) TQ_SM(2, 3) TQ_SM(2, 4) TQ_SM(3, 2) TQ_SM(3, 3) TQ_SM(3, 4)
  TQ_SM(4, 2) TQ_SM(4, 3) TQ_SM(4, 4)
#undef TQ_SM
}

// -----------------------------------------------------------------------------------------
// Decode for every other head_dim (a multiple of 8 up to 256; the TurboQuant page's
// vector-search section uses d = 200): the direct kernel's structure with d, the code widths
// and the sketch width read at run time.  One workgroup per (chunk of kGenTok tokens, KV head,
// sequence): the chunk's records are copied into LDS as words, the codes unpacked from there
// (field_code: 1/2/4-bit codes a little-endian bitstream, 3-bit codes in groups of 32 per 12
// bytes with a trailing partial group as a plain bitstream), then every (token, head)
// estimate, the chunk's softmax and every (head, coordinate) output, as decode_small_kernel.
// -----------------------------------------------------------------------------------------
constexpr int kDecGenTok = 32, kDecGenMaxM = 256, kDecGenMaxRec = 4 * kGenRecWords;

// Code j of a field of n codes of width b, from the field's bytes.  May read one byte past the
// field's last code, which stays inside the record (another field, the norms or the pad).
__device__ __forceinline__ uint32_t field_code(const uint8_t* f, int j, int b, int n) {
  const int whole = b == 3 ? (n & ~31) : 0;
  if (j < whole) {
    const uint8_t* g = f + 12 * (j >> 5);
    const uint32_t w0 = g[0] | (g[1] << 8) | (g[2] << 16) | ((uint32_t)g[3] << 24);
    const uint32_t w1 = g[4] | (g[5] << 8) | (g[6] << 16) | ((uint32_t)g[7] << 24);
    const uint32_t w2 = g[8] | (g[9] << 8) | (g[10] << 16) | ((uint32_t)g[11] << 24);
    return group3_code(w0, w1, w2, j & 31);
  }
  const uint8_t* base = f + (whole >> 5) * 12;
  const int pos = b * (j - whole);
  const uint32_t v = (uint32_t)base[pos >> 3] | ((uint32_t)base[(pos >> 3) + 1] << 8);
  return (v >> (pos & 7)) & ((1u << b) - 1u);
}

__global__ __launch_bounds__(kSmallThreads) void decode_generic_kernel(DecodeArgs A) {
  __shared__ float qx[kSmallMaxG][kGenMaxD + 1];
  __shared__ float qs[kSmallMaxG][kDecGenMaxM + 1];
  __shared__ __attribute__((aligned(16))) uint32_t raw[kDecGenTok][kDecGenMaxRec / 4];
  __shared__ uint8_t kc[kDecGenTok][kGenMaxD];
  __shared__ uint8_t vc[kDecGenTok][kGenMaxD];
  __shared__ uint8_t sb[kDecGenTok][kDecGenMaxM];
  __shared__ float nr[kDecGenTok][3];
  __shared__ int ok_t[kDecGenTok];
  __shared__ float lg[kSmallMaxG][kDecGenTok + 1];
  __shared__ float hm[kSmallMaxG], hl[kSmallMaxG];
  __shared__ float kl[kMaxLevels], vl[kMaxLevels];
  const int G = A.G, m = A.m, d = A.d, TOK = A.chunk, tid = threadIdx.x;
  const int b = blockIdx.z, hkv = blockIdx.y, chunk = blockIdx.x;
  const int64_t qrow0 = (int64_t)b * A.q_heads + (int64_t)hkv * G;
  if (A.gate) {
    bool any = false;
    for (int j = 0; j < G; ++j) any = any || A.gate[qrow0 + j] != 0;
    if (!any) return;
  }
  const bool gather = A.sel_idx != nullptr;
  const int n = gather ? A.k_sel : (int)min((int64_t)A.seq_lens[b], A.capacity);
  const int c0 = chunk * TOK, nt = max(0, min(TOK, n - c0));
  const uint8_t* recs = A.records + ((int64_t)b * A.kv_heads + hkv) * A.capacity * A.rec_bytes;
  for (int e = tid; e < G * d; e += kSmallThreads) qx[e / d][e % d] = A.qx[(qrow0 + e / d) * d + e % d];
  for (int e = tid; e < G * m; e += kSmallThreads) qs[e / m][e % m] = A.qs[(qrow0 + e / m) * m + e % m];
  if (tid < kMaxLevels) {
    kl[tid] = A.key_levels[tid];
    vl[tid] = A.val_levels[tid];
  }
  // the chunk's records as words (records are 16-byte multiples)
  const int rw = A.rec_bytes / 4;
  for (int e = tid; e < nt * rw; e += kSmallThreads) {
    const int t = e / rw, w = e % rw;
    int64_t tok = c0 + t;
    bool ok = true;
    if (gather) {
      tok = A.sel_idx[((int64_t)b * A.kv_heads + hkv) * A.k_sel + c0 + t];
      ok = tok >= 0 && tok < A.capacity;
    }
    raw[t][w] = reinterpret_cast<const uint32_t*>(recs + (ok ? tok : 0) * A.rec_bytes)[w];
    if (w == 0) ok_t[t] = ok ? 1 : 0;
  }
  __syncthreads();
  const int per_t = 2 * d + m;
  for (int e = tid; e < nt * per_t; e += kSmallThreads) {
    const int t = e / per_t, j = e % per_t;
    const uint8_t* r = reinterpret_cast<const uint8_t*>(raw[t]);
    if (j < d) kc[t][j] = (uint8_t)field_code(r, j, A.kb, d);
    else if (j < 2 * d) vc[t][j - d] = (uint8_t)field_code(r + A.kbytes + A.sbytes, j - d, A.vb, d);
    else sb[t][j - 2 * d] = (uint8_t)((r[A.kbytes + ((j - 2 * d) >> 3)] >> ((j - 2 * d) & 7)) & 1u);
  }
  for (int t = tid; t < nt; t += kSmallThreads) {
    const float* f = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(raw[t]) + A.norm_off);
    nr[t][0] = f[0];
    nr[t][1] = f[1];
    nr[t][2] = f[2];
  }
  __syncthreads();
  const int items = nt * G;
  int L = 1;
  while (L < 8 && items * L * 2 <= kSmallThreads) L *= 2;
  for (int i0 = 0; i0 < items; i0 += kSmallThreads / L) {
    const int it = i0 + tid / L, s = tid % L;
    const int t = it / G, h = it % G;
    float dot = 0.0f, qd = 0.0f;
    if (it < items) {
      for (int i = s; i < d; i += L) dot = fmaf(qx[h][i], kl[kc[t][i]], dot);
      for (int j = s; j < m; j += L) qd += sb[t][j] ? qs[h][j] : -qs[h][j];
    }
    for (int msk = 1; msk < L; msk <<= 1) {
      dot += __shfl_xor(dot, msk);
      qd += __shfl_xor(qd, msk);
    }
    if (it < items && s == 0) {
      const float logit = ok_t[t] ? A.scale * fmaf(A.qjl_coef * nr[t][1], qd, nr[t][0] * A.inv_sqrt_d * dot)
                                  : kNegInf;
      lg[h][t] = logit;
      if (A.logits && ok_t[t]) A.logits[(qrow0 + h) * A.logit_stride + c0 + t] = logit;
    }
  }
  __syncthreads();
  for (int h = tid; h < G; h += kSmallThreads) {
    float mx = kNegInf;
    for (int t = 0; t < nt; ++t) mx = fmaxf(mx, lg[h][t]);
    float l = 0.0f;
    for (int t = 0; t < nt; ++t) {
      const float p = (mx == kNegInf || lg[h][t] == kNegInf) ? 0.0f : __expf(lg[h][t] - mx);
      l += p;
      lg[h][t] = p * nr[t][2] * A.inv_sqrt_d;
    }
    hm[h] = mx;
    hl[h] = l;
  }
  __syncthreads();
  const int stride = d + 2;
  for (int e = tid; e < G * d; e += kSmallThreads) {
    const int h = e / d, i = e % d;
    float o = 0.0f;
    for (int t = 0; t < nt; ++t) o = fmaf(lg[h][t], vl[vc[t][i]], o);
    A.part[((qrow0 + h) * A.n_chunks + chunk) * stride + 2 + i] = o;
  }
  for (int h = tid; h < G; h += kSmallThreads) {
    A.part[((qrow0 + h) * A.n_chunks + chunk) * stride] = hm[h];
    A.part[((qrow0 + h) * A.n_chunks + chunk) * stride + 1] = hl[h];
  }
}

// -----------------------------------------------------------------------------------------
// Matrix-core decode scan for head_dim 128 and 4 query heads per KV head (2- or 3-bit keys,
// 4-bit values).  Same arithmetic as decode_scan_kernel, laid out for gfx950.  Each wave
// takes 16 tokens per step:
//  * key scores on v_mfma_i32_16x16x64_i8, exact in int32: rows = (head, part), columns =
//    tokens.  Key levels are two-limb fixed point (level ~= (256 hi + lo) / F with int8 limbs,
//    F chosen on the host so the levels sit near integers); queries and query sketches are
//    three-limb fixed point (24 bits against the head's largest entry).  The code product
//    keeps the limb products of weight 2^24, 2^16 and 2^8 (three rows per head) and drops
//    only low x low (2^-24 relative); the QJL product has its own accumulator with one row
//    per sketch limb.  Level limbs come from registers (v_perm_b32, 4 codes per
//    instruction); QJL bits enter as 0/1 bytes and the sketch sum is subtracted afterwards.
//    Lane (kg, n) receives every part of head kg for token n and combines them in registers;
//  * the running maximum of each head is shared by its 16 lanes (raised lazily), p and
//    w = p r_v / sqrt(d) per lane;
//  * value aggregation on v_mfma_f32_16x16x32_bf16: rows = coordinates, K = (token, level
//    half), columns = (head, w half); the 16 tokens' value codes are transposed through 1 KB
//    of LDS and their level halves read as pairs from a 16-entry LDS table.
// -----------------------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// A 16-byte store marked non-temporal: output written once and not read back by the kernel
// (the bulk scans' score matrices), so it streams out instead of displacing cached inputs.
__device__ __forceinline__ void nt_store4(float* dst, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Two int8 limbs of a fixed-point integer v (|v| <= 32639): v = 256 hi + lo, lo in [-128, 127].
__device__ __forceinline__ void int8_limbs(int v, int& hi, int& lo) {
  hi = (v + 128) >> 8;
  lo = v - 256 * hi;
}
// Three int8 limbs (|v| <= 127 * 65536 + 32767): v = 65536 l2 + 256 l1 + l0, l0, l1 in [-128, 127].
__device__ __forceinline__ void int8_limbs3(int v, int& l2, int& l1, int& l0) {
  int rest;
  int8_limbs(v, rest, l0);
  int8_limbs(rest, l2, l1);
}

// Coordinate (within a lane's 32-coordinate slice) of byte k of key selector s.  3-bit codes:
// selector s holds codes 4s .. 4s+3 (a masked word of the 32-code group layout); 2-bit codes:
// selector 4w + t holds the codes at bits 2t of every byte of word w, i.e. 16w + 4k + t.
template <int BK>
__device__ constexpr int sel_coord(int s, int k) {
  return BK == 3 ? 4 * s + k : 16 * (s >> 2) + 4 * k + (s & 3);
}

__device__ __forceinline__ uint32_t bf16_rn_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_bits_f(uint32_t h) { return __uint_as_float(h << 16); }
// high (sp = 0) or low (sp = 1) bf16 half of x: x ~= hi + lo with ~16 significant bits
__device__ __forceinline__ uint32_t bf16_half(float x, int sp) {
  const uint32_t hi = bf16_rn_bits(x);
  return sp == 0 ? hi : bf16_rn_bits(x - bf16_bits_f(hi));
}
__device__ __forceinline__ uint32_t bf16_pair(float x) {      // hi | lo << 16
  const uint32_t hi = bf16_rn_bits(x);
  return hi | (bf16_rn_bits(x - bf16_bits_f(hi)) << 16);
}

// Per (sequence, KV head) preparation for the matrix-core scan: q_x = Pi q and q_s = (S Pi) q
// for the group's G query heads in one pass (float64 sums rounded once to float32; thread
// (row o, slice) holds 16 coordinates of row o of Pi and of S Pi, loaded up front), then the lanes' query
// operands: bop[group][lane][32 words] = code words (16), QJL words (8), and the scales of lane
// L's head L / 16, {1 / (F_q F_k), 2 / F_s, -sum / F_s} (3), pad.
// SCAN: the B operands of the bulk scan's 16-token x 16-query tiles, for a group of 4
// consecutive queries of one (sequence, KV head) (q_heads = queries per unit, kv_heads = groups
// per unit, a multiple of 4; rows past the last query are zero).  Group g supplies columns
// 4 (g % 4) .. + 3 of query tile g / 4, stored chunk-major: bop[tile][chunk][lane][4 words],
// lane L = (query column L % 16, K slice kg = L / 16):
//   chunks 0..5: limb 2 - c / 2 of the fixed-point q_x, K chunk c % 2 (word w, byte k <->
//     coordinate 32 kg + sel_coord(4 (c % 2) + w, k), as the token side's selectors);
//   chunks 6..11: limb 2 - (c - 6) / 2 of the fixed-point q_s, bit chunk (c - 6) % 2 (word w,
//     byte k <-> sketch coordinate 32 kg + 8 k + 4 ((c - 6) % 2) + w);
//   chunk 12: {1 / (F_q F_k), 2 / F_s, -sum / F_s, 0} of the column's query (fk = F_k, the
//     three-limb key level scale).
constexpr int kScanChunks = 13;      // bulk-scan operand chunks (16 B per lane) per query tile

constexpr int kPrepThreads = 1024;
// POLAR (decode only): no key chunks; the QJL chunks 0, 1 and the scales (the first is 2^e,
// e the head's power of two above max |q_x|) as above, 12 words per lane, and q_x itself in
// float32 to qx_out [rows][128] (the decode builds its per-query pair tables from it).
constexpr int kPolarLaneWords = 12;

template <int BK, bool QJL, bool SCAN, bool POLAR = false>
__global__ __launch_bounds__(kPrepThreads) void mfma_prep_kernel(const float* __restrict__ pi,
                                                                 const float* __restrict__ s_pi, const void* q,
                                                                 tq_dtype q_dt, int q_heads, int kv_heads,
                                                                 float fk, uint32_t* bop, float* qx_out) {
  constexpr int D = 128, G = 4;
  __shared__ double qv[G][D];
  __shared__ __attribute__((aligned(16))) float xf[G][D], sf[G][D];
  const int group = blockIdx.x, b = group / kv_heads, hkv = group % kv_heads;
  const int64_t qrow0 = (int64_t)b * q_heads + (int64_t)hkv * G;
  const int rows = SCAN ? min(G, q_heads - hkv * G) : G;
  // thread (row o, slice ks): coordinates 32 jj + 4 ks .. + 3 (jj < 4) of row o of Pi and of
  // S Pi against the group's G queries, so that the eight lanes of a row read whole 128-byte
  // lines; the eight slices are summed across adjacent lanes
  const int o = threadIdx.x >> 3, ks = threadIdx.x & 7;
  float4 wp[4], ws[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    wp[jj] = *reinterpret_cast<const float4*>(pi + o * D + 32 * jj + 4 * ks);
    if (QJL) ws[jj] = *reinterpret_cast<const float4*>(s_pi + o * D + 32 * jj + 4 * ks);
  }
  if (threadIdx.x < G * D) {
    const int h = threadIdx.x / D, i = threadIdx.x % D;
    qv[h][i] = h < rows ? (double)load_elem(q, q_dt, (qrow0 + h) * D + i) : 0.0;
  }
  __syncthreads();
  {
    double ax[G], as[G];
#pragma unroll
    for (int h = 0; h < G; ++h) ax[h] = as[h] = 0.0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const double* vv = qv[h] + 32 * jj + 4 * ks;
        ax[h] = fma((double)wp[jj].x, vv[0], ax[h]);
        ax[h] = fma((double)wp[jj].y, vv[1], ax[h]);
        ax[h] = fma((double)wp[jj].z, vv[2], ax[h]);
        ax[h] = fma((double)wp[jj].w, vv[3], ax[h]);
        if (QJL) {
          as[h] = fma((double)ws[jj].x, vv[0], as[h]);
          as[h] = fma((double)ws[jj].y, vv[1], as[h]);
          as[h] = fma((double)ws[jj].z, vv[2], as[h]);
          as[h] = fma((double)ws[jj].w, vv[3], as[h]);
        }
      }
#pragma unroll
    for (int msk = 1; msk < 8; msk <<= 1)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        ax[h] += __shfl_xor(ax[h], msk);
        if (QJL) as[h] += __shfl_xor(as[h], msk);
      }
    if (ks == 0)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        xf[h][o] = (float)ax[h];
        sf[h][o] = (float)as[h];
        if (POLAR) qx_out[(qrow0 + h) * D + o] = (float)ax[h];   // the decode's pair tables
      }
  }
  __syncthreads();
  // per head: fixed-point scales (three int8 limbs against the largest |entry|) and the sum of
  // the sketch's fixed-point values
  __shared__ float s_fq[G], s_fs[G], s_pe[G];
  __shared__ int s_ssum[G];
  if (threadIdx.x < G * 64) {
    const int h = threadIdx.x >> 6, l = threadIdx.x & 63;   // wave h reduces head h
    float mx = fmaxf(fabsf(xf[h][l]), fabsf(xf[h][l + 64]));
    float ms = QJL ? fmaxf(fabsf(sf[h][l]), fabsf(sf[h][l + 64])) : 0.0f;
#pragma unroll
    for (int msk = 32; msk > 0; msk >>= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, msk));
      ms = fmaxf(ms, __shfl_xor(ms, msk));
    }
    constexpr float kFix3 = 8323072.0f;   // 127 * 65536: the three-limb range
    const float fq = mx > 0.0f ? kFix3 / mx : 1.0f, fs = ms > 0.0f ? kFix3 / ms : 1.0f;
    int ss = QJL ? (int)rintf(sf[h][l] * fs) + (int)rintf(sf[h][l + 64] * fs) : 0;
#pragma unroll
    for (int msk = 32; msk > 0; msk >>= 1) ss += __shfl_xor(ss, msk);
    if (l == 0) {
      s_fq[h] = fq;
      s_fs[h] = fs;
      s_ssum[h] = ss;
      int e = 0;
      if (mx > 0.0f) frexpf(mx, &e);          // mx < 2^e
      s_pe[h] = (float)e;
    }
  }
  __syncthreads();
  // the three int8 limbs of every fixed-point query coordinate and sketch coordinate, formed
  // once and packed as bytes (l2, l1, l0, 0); coordinate i of head h at h LS + i + i / 32, so
  // that the 16 (head, K slice) addresses of an operand read below fall on distinct banks.
  // A sketch coordinate c carries its in-place bit weight s = c % 8 (decode).
  constexpr int LS = D + 4;
  __shared__ uint32_t klimb[POLAR ? 1 : G * LS], jlimb[QJL ? G * LS : 1];
  if constexpr (!POLAR || QJL) {
    const int h = (threadIdx.x >> 7) & 3, i = threadIdx.x & 127, at = h * LS + i + (i >> 5);
    int l2, l1, l0;
    if (threadIdx.x < G * D) {
      if constexpr (!POLAR) {
        int8_limbs3((int)rintf(xf[h][i] * s_fq[h]), l2, l1, l0);
        klimb[at] = (uint32_t)(l2 & 0xFF) | (uint32_t)(l1 & 0xFF) << 8 | (uint32_t)(l0 & 0xFF) << 16;
      }
    } else if (QJL) {
      const int s = i & 7;
      const float sv = sf[h][i] * s_fs[h];
      const int qv = SCAN ? (int)rintf(sv) : s == 7 ? -(int)rintf(sv * 0.0078125f)
                                                     : (int)rintf(sv * (1.0f / (float)(1 << s)));
      int8_limbs3(qv, l2, l1, l0);
      jlimb[at] = (uint32_t)(l2 & 0xFF) | (uint32_t)(l1 & 0xFF) << 8 | (uint32_t)(l0 & 0xFF) << 16;
    }
    __syncthreads();
  }
  if constexpr (SCAN) {
    // 13 chunks x 16 lanes (this group's 4 columns x 4 K slices), one 16-byte word each
    const int t = threadIdx.x;
    if (t >= kScanChunks * 16) return;
    const int c = t >> 4, h = (t >> 2) & 3, kg = t & 3;
    const int L = 4 * (group & 3) + h + 16 * kg;   // kv_heads % 4 == 0: group % 4 = column block
    u32x4 words = u32x4{0u, 0u, 0u, 0u};
    if (c < 6) {
      const int bi = c >> 1, hh = c & 1;          // byte bi of a packed word = limb 2 - bi
      const uint32_t* kl = klimb + h * LS + 33 * kg;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) word |= ((kl[sel_coord<BK>(4 * hh + w, k)] >> (8 * bi)) & 0xFFu) << (8 * k);
        words[w] = word;
      }
    } else if (c < 12) {
      if (QJL) {
        const int bi = (c - 6) >> 1, jj = (c - 6) & 1;
        const uint32_t* jl = jlimb + h * LS + 33 * kg;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t word = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) word |= ((jl[8 * k + 4 * jj + w] >> (8 * bi)) & 0xFFu) << (8 * k);
          words[w] = word;
        }
      }
    } else {
      const float bk = 1.0f / (s_fq[h] * fk);
      const float bq = QJL ? 2.0f / s_fs[h] : 0.0f;
      const float oq = QJL ? -(float)s_ssum[h] / s_fs[h] : 0.0f;
      words = u32x4{__float_as_uint(bk), __float_as_uint(bq), __float_as_uint(oq), 0u};
    }
    reinterpret_cast<u32x4*>(bop)[((int64_t)(group >> 2) * kScanChunks + c) * 64 + L] = words;
    return;
  }
  // operand words (A of the score products): lane L = (row n = L % 16, K slice kg = L / 16),
  // head n / 4, part n % 4.
  //  code word (j, w): byte k <-> coordinate 32 kg + sel_coord(2j + (w & 1), k); w < 2: high
  //    level limb slots, w >= 2: low limb slots.  part 0 (weight 2^24): hi x q2; part 1 (2^16):
  //    hi x q1 + lo x q2; part 2 (2^8): hi x q0 + lo x q1; part 3: zero.
  //  QJL word (j, w): byte k <-> sketch coordinate 32 kg + 8k + 4j + w; part p < 3 holds limb
  //    2 - p of the sketch (weight 2^(8 (2 - p))); part 3: zero.
  // one 16-byte chunk per wave (no divergence): waves 0 .. NC - 1 the code chunks, the next two
  // the QJL chunks, the next one the scales, each for lane L = its own lane
  constexpr int NC = POLAR ? 0 : 4;
  const int L = threadIdx.x & 63, role = threadIdx.x >> 6;
  if (role > NC + 2) return;
  const int n = L & 15, kg = L >> 4, hB = n >> 2, part = n & 3;
  u32x4* gdst = reinterpret_cast<u32x4*>(
      bop + ((int64_t)group * 64 + L) * (POLAR ? kPolarLaneWords : 32));
  if (role < NC) {
    // byte b of a packed limb word: 0 = l2, 1 = l1, 2 = l0, 3 = zero
    const int j = role;
    const uint32_t* kl = klimb + hB * LS + 33 * kg;
    u32x4 words;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // high level limb slots (w < 2): part p takes query limb 2 - p; low slots: limb 3 - p
      const bool hi_slot = w < 2;
      const int bi = part == 0 ? (hi_slot ? 0 : 3) : part == 1 ? (hi_slot ? 1 : 0) : part == 2 ? (hi_slot ? 2 : 1) : 3;
      uint32_t word = 0;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int coord = sel_coord<BK>(2 * j + (w & 1), kk);
        word |= ((kl[coord] >> (8 * bi)) & 0xFFu) << (8 * kk);
      }
      words[w] = word;
    }
    gdst[j] = words;
  } else if (role < NC + 2) {
    // decode: the token side holds bit s = 4 j + w of each sketch byte in place (byte value
    // 2^s b, -128 b for s = 7), so this side holds the sketch scaled by 2^-s (negated for
    // s = 7); part p < 3 takes limb 2 - p, i.e. byte p of the packed word
    const int j = role - NC;
    const uint32_t* jl = jlimb + hB * LS + 33 * kg;
    u32x4 words;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
      if (QJL)
#pragma unroll
        for (int k = 0; k < 4; ++k) word |= ((jl[8 * k + 4 * j + w] >> (8 * part)) & 0xFFu) << (8 * k);
      words[w] = word;
    }
    gdst[NC + j] = words;
  } else {
    // the score lanes of head / query kg combine its parts with these
    const float fqk = s_fq[kg], fsk = s_fs[kg];
    const float bk = POLAR ? ldexpf(1.0f, (int)s_pe[kg]) : 1.0f / (fqk * fk);
    const float bq = QJL ? 2.0f / fsk : 0.0f;
    const float oq = QJL ? -(float)s_ssum[kg] / fsk : 0.0f;
    gdst[NC + 2] = u32x4{__float_as_uint(bk), __float_as_uint(bq), __float_as_uint(oq), 0u};
  }
}

// Per (sequence, KV head, query head of the group) preparation for the matrix-core decode with
// scalar key codes: the same operands as mfma_prep_kernel<BK, QJL, false>, one head per block so
// that four times as many blocks each carry a quarter of the work (q_x = Pi q and q_s = (S Pi) q
// in float64 rounded once to float32, the head's fixed-point scales, its int8 limbs, then the
// operand chunks of its 16 lanes (row n = 4 h .. 4 h + 3) and the scale chunk of the 16 lanes of
// K slice h).
template <int BK, bool QJL>
__global__ __launch_bounds__(kPrepThreads) void mfma_prep_head_kernel(const float* __restrict__ pi,
                                                                      const float* __restrict__ s_pi,
                                                                      const void* q, tq_dtype q_dt, int q_heads,
                                                                      int kv_heads, float fk, uint32_t* bop) {
  constexpr int D = 128, G = 4, LS = D + D / 32;
  __shared__ double qv[D];
  __shared__ float xf[D], sf[D];
  __shared__ float s_fq, s_fs;
  __shared__ int s_ssum;
  __shared__ uint32_t klimb[LS], jlimb[QJL ? LS : 1];
  const int group = blockIdx.x >> 2, h = blockIdx.x & 3, b = group / kv_heads, hkv = group % kv_heads;
  const int64_t qrow = (int64_t)b * q_heads + (int64_t)hkv * G + h;
  // thread (row o, slice ks): coordinates 32 jj + 4 ks .. + 3 of row o of Pi and of S Pi, so
  // that the eight lanes of a row read whole 128-byte lines
  const int o = threadIdx.x >> 3, ks = threadIdx.x & 7;
  float4 wp[4], ws[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    wp[jj] = *reinterpret_cast<const float4*>(pi + o * D + 32 * jj + 4 * ks);
    if (QJL) ws[jj] = *reinterpret_cast<const float4*>(s_pi + o * D + 32 * jj + 4 * ks);
  }
  if (threadIdx.x < D) qv[threadIdx.x] = (double)load_elem(q, q_dt, qrow * D + threadIdx.x);
  __syncthreads();
  {
    double ax = 0.0, as = 0.0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const double* vv = qv + 32 * jj + 4 * ks;
      ax = fma((double)wp[jj].x, vv[0], ax);
      ax = fma((double)wp[jj].y, vv[1], ax);
      ax = fma((double)wp[jj].z, vv[2], ax);
      ax = fma((double)wp[jj].w, vv[3], ax);
      if (QJL) {
        as = fma((double)ws[jj].x, vv[0], as);
        as = fma((double)ws[jj].y, vv[1], as);
        as = fma((double)ws[jj].z, vv[2], as);
        as = fma((double)ws[jj].w, vv[3], as);
      }
    }
#pragma unroll
    for (int msk = 1; msk < 8; msk <<= 1) {
      ax += __shfl_xor(ax, msk);
      if (QJL) as += __shfl_xor(as, msk);
    }
    if (ks == 0) {
      xf[o] = (float)ax;
      sf[o] = (float)as;
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // fixed-point scales (three int8 limbs against the largest |entry|) and the sum of the
    // sketch's fixed-point values
    const int l = threadIdx.x;
    float mx = fmaxf(fabsf(xf[l]), fabsf(xf[l + 64]));
    float ms = QJL ? fmaxf(fabsf(sf[l]), fabsf(sf[l + 64])) : 0.0f;
#pragma unroll
    for (int msk = 32; msk > 0; msk >>= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, msk));
      ms = fmaxf(ms, __shfl_xor(ms, msk));
    }
    constexpr float kFix3 = 8323072.0f;   // 127 * 65536: the three-limb range
    const float fq = mx > 0.0f ? kFix3 / mx : 1.0f, fs = ms > 0.0f ? kFix3 / ms : 1.0f;
    int ss = QJL ? (int)rintf(sf[l] * fs) + (int)rintf(sf[l + 64] * fs) : 0;
#pragma unroll
    for (int msk = 32; msk > 0; msk >>= 1) ss += __shfl_xor(ss, msk);
    if (l == 0) {
      s_fq = fq;
      s_fs = fs;
      s_ssum = ss;
    }
  }
  __syncthreads();
  // the three int8 limbs of every fixed-point query and sketch coordinate, packed as bytes
  // (l2, l1, l0, 0); coordinate i at i + i / 32 (the 4 K-slice addresses of a read fall on
  // distinct banks).  A sketch coordinate c carries its in-place bit weight s = c % 8.
  if (threadIdx.x < 2 * D) {
    const int i = threadIdx.x & (D - 1), at = i + (i >> 5);
    int l2, l1, l0;
    if (threadIdx.x < D) {
      int8_limbs3((int)rintf(xf[i] * s_fq), l2, l1, l0);
      klimb[at] = (uint32_t)(l2 & 0xFF) | (uint32_t)(l1 & 0xFF) << 8 | (uint32_t)(l0 & 0xFF) << 16;
    } else if (QJL) {
      const int s = i & 7;
      const float sv = sf[i] * s_fs;
      int8_limbs3(s == 7 ? -(int)rintf(sv * 0.0078125f) : (int)rintf(sv * (1.0f / (float)(1 << s))), l2, l1, l0);
      jlimb[at] = (uint32_t)(l2 & 0xFF) | (uint32_t)(l1 & 0xFF) << 8 | (uint32_t)(l0 & 0xFF) << 16;
    }
  }
  __syncthreads();
  // 16 threads per 16-byte chunk: roles 0..3 the code chunks and 4, 5 the QJL chunks of lanes
  // (row n = 4 h + part, K slice kg); role 6 the scale chunk of lanes (row n, K slice h)
  const int role = threadIdx.x >> 4, idx = threadIdx.x & 15;
  if (role > 6) return;
  const int part = idx & 3, kg = role < 6 ? idx >> 2 : h, n = role < 6 ? 4 * h + part : idx;
  u32x4* gdst = reinterpret_cast<u32x4*>(bop + ((int64_t)group * 64 + n + 16 * kg) * 32);
  if (role < 4) {
    // byte bi of a packed limb word: 0 = l2, 1 = l1, 2 = l0, 3 = zero.  High level limb slots
    // (w < 2): part p takes query limb 2 - p; low slots: limb 3 - p
    const uint32_t* kl = klimb + 33 * kg;
    u32x4 words;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bool hi_slot = w < 2;
      const int bi = part == 0 ? (hi_slot ? 0 : 3) : part == 1 ? (hi_slot ? 1 : 0) : part == 2 ? (hi_slot ? 2 : 1) : 3;
      uint32_t word = 0;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) word |= ((kl[sel_coord<BK>(2 * role + (w & 1), kk)] >> (8 * bi)) & 0xFFu) << (8 * kk);
      words[w] = word;
    }
    gdst[role] = words;
  } else if (role < 6) {
    // the token side holds bit s = 4 j + w of each sketch byte in place; part p < 3 takes
    // limb 2 - p, i.e. byte p of the packed word
    const int j = role - 4;
    const uint32_t* jl = jlimb + 33 * kg;
    u32x4 words;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
      if (QJL)
#pragma unroll
        for (int k = 0; k < 4; ++k) word |= ((jl[8 * k + 4 * j + w] >> (8 * part)) & 0xFFu) << (8 * k);
      words[w] = word;
    }
    gdst[role] = words;
  } else {
    const float bq = QJL ? 2.0f / s_fs : 0.0f, oq = QJL ? -(float)s_ssum / s_fs : 0.0f;
    gdst[6] = u32x4{__float_as_uint(1.0f / (s_fq * fk)), __float_as_uint(bq), __float_as_uint(oq), 0u};
  }
}

// Merge without an exact segment, one block per (sequence, KV head): the GG query heads of the
// group share one read of Pi^T (D / 2 entries per thread, applied to all GG vectors).
// 256 threads; rows row0 .. row0 + GG - 1 of part [rows][nch][D + 2] = (m, l, o_x[D]) in, out
// [rows][D] and lse [rows] (if not NULL) out.
template <int D, int GG>
__device__ __forceinline__ void merge_group(const float* __restrict__ pi_t, const float* part,
                                            float* out, float* lse, int64_t row0, int nch) {
  __shared__ __attribute__((aligned(16))) float ox[GG][D];
  __shared__ float sM[GG], sL[GG];
  constexpr int stride = D + 2;
  // thread (slice ks, rows orow + (256 / 8) r): coordinates 32 jj + 4 ks .. + 3 (jj < D / 32)
  // of D / 32 rows of Pi^T, loaded up front so that eight lanes read whole 128-byte lines
  constexpr int NJ = D / 32, RS = 256 / 8, NR = D / RS;
  const int ks = threadIdx.x & 7, orow = threadIdx.x >> 3;
  float4 w[NR][NJ];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
      w[r][jj] = *reinterpret_cast<const float4*>(pi_t + (int64_t)(orow + RS * r) * D + 32 * jj + 4 * ks);
  // rotated-domain output of head h, coordinate i
  constexpr int PER = (GG * D + 255) / 256;   // elements per thread
  constexpr int SPLIT = GG * D <= 128 ? 256 / (GG * D) : 1;   // threads per element (many chunks)
  __shared__ float spl[SPLIT][SPLIT > 1 ? GG * D : 1], spM[SPLIT][GG], spL[SPLIT][GG];
  if (nch <= 8) {
    // one memory round trip: every chunk's (m, l, o_i) of this thread's elements at once
    float mc[PER][8], lc[PER][8], ov[PER][8];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = min((int)threadIdx.x + 256 * p, GG * D - 1), h = e / D, i = e % D;
      const float* pr = part + (row0 + h) * nch * stride;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int cc = min(u, nch - 1);
        mc[p][u] = u < nch ? pr[(int64_t)cc * stride] : kNegInf;
        lc[p][u] = pr[(int64_t)cc * stride + 1];
        ov[p][u] = pr[(int64_t)cc * stride + 2 + i];
      }
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = (int)threadIdx.x + 256 * p;
      if (e >= GG * D) break;
      const int h = e / D, i = e % D;
      float M = kNegInf;
#pragma unroll
      for (int u = 0; u < 8; ++u) M = fmaxf(M, mc[p][u]);
      float L = 0.0f, acc = 0.0f;
      if (M != kNegInf) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wgt = mc[p][u] == kNegInf ? 0.0f : __expf(mc[p][u] - M);
          acc = fmaf(ov[p][u], wgt, acc);
          L = fmaf(lc[p][u], wgt, L);
        }
      }
      ox[h][i] = acc;
      if (i == 0) {
        sM[h] = M;
        sL[h] = L;
      }
    }
  } else if (SPLIT > 1 && nch <= 16 * SPLIT) {
    // SPLIT threads per element, each over 16 strided chunks in one memory round trip (a chunk
    // with m = -inf weighs 0), then the SPLIT partial sums combined through LDS
    const int e = (int)threadIdx.x % (GG * D), sp = (int)threadIdx.x / (GG * D), h = e / D, i = e % D;
    const float* pr = part + (row0 + h) * nch * stride;
    float mc[16], lc[16], ov[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int c = sp + SPLIT * u, cc = min(c, nch - 1);
      mc[u] = c < nch ? pr[(int64_t)cc * stride] : kNegInf;
      lc[u] = pr[(int64_t)cc * stride + 1];
      ov[u] = pr[(int64_t)cc * stride + 2 + i];
    }
    float M = kNegInf;
#pragma unroll
    for (int u = 0; u < 16; ++u) M = fmaxf(M, mc[u]);
    float L = 0.0f, acc = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float wgt = mc[u] == kNegInf ? 0.0f : __expf(mc[u] - M);
        acc = fmaf(ov[u], wgt, acc);
        L = fmaf(lc[u], wgt, L);
      }
    }
    spl[sp][e] = acc;
    if (i == 0) {
      spM[sp][h] = M;
      spL[sp][h] = L;
    }
    __syncthreads();
    if ((int)threadIdx.x < GG * D) {
      float Mt = kNegInf;
#pragma unroll
      for (int s2 = 0; s2 < SPLIT; ++s2) Mt = fmaxf(Mt, spM[s2][h]);
      float Lt = 0.0f, at = 0.0f;
      if (Mt != kNegInf) {
#pragma unroll
        for (int s2 = 0; s2 < SPLIT; ++s2) {
          const float wgt = spM[s2][h] == kNegInf ? 0.0f : __expf(spM[s2][h] - Mt);
          at = fmaf(spl[s2][e], wgt, at);
          Lt = fmaf(spL[s2][h], wgt, Lt);
        }
      }
      ox[h][i] = at;
      if (i == 0) {
        sM[h] = Mt;
        sL[h] = Lt;
      }
    }
  } else {
  // one pass over the chunk partials with a running maximum (eight chunks' loads in flight at a
  // time; a chunk with m = -inf weighs 0); every thread of a head forms the same maximum and
  // weight sum
  for (int e = threadIdx.x; e < GG * D; e += blockDim.x) {
    const int h = e / D, i = e % D;
    const float* pr = part + (row0 + h) * nch * stride;
    float M = kNegInf, L = 0.0f, acc = 0.0f;
    for (int c = 0; c < nch; c += 8) {
      float mc[8], lc[8], ov[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int cc = min(c + u, nch - 1);
        mc[u] = c + u < nch ? pr[(int64_t)cc * stride] : kNegInf;
        lc[u] = pr[(int64_t)cc * stride + 1];
        ov[u] = pr[(int64_t)cc * stride + 2 + i];
      }
      float Mn = M;
#pragma unroll
      for (int u = 0; u < 8; ++u) Mn = fmaxf(Mn, mc[u]);
      if (Mn == kNegInf) continue;
      const float sc = M == kNegInf ? 0.0f : __expf(M - Mn);
      acc *= sc;
      L *= sc;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wgt = mc[u] == kNegInf ? 0.0f : __expf(mc[u] - Mn);
        acc = fmaf(ov[u], wgt, acc);
        L = fmaf(lc[u], wgt, L);
      }
      M = Mn;
    }
    ox[h][i] = acc;
    if (i == 0) {
      sM[h] = M;
      sL[h] = L;
    }
  }
  }
  __syncthreads();
  // o = Pi^T o_x / L for the GG heads
#pragma unroll
  for (int h = 0; h < GG; ++h) {
    float acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const float4 xv = *reinterpret_cast<const float4*>(ox[h] + 32 * jj + 4 * ks);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        acc[r] = fmaf(w[r][jj].x, xv.x, acc[r]);
        acc[r] = fmaf(w[r][jj].y, xv.y, acc[r]);
        acc[r] = fmaf(w[r][jj].z, xv.z, acc[r]);
        acc[r] = fmaf(w[r][jj].w, xv.w, acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int msk = 1; msk < 8; msk <<= 1) acc[r] += __shfl_xor(acc[r], msk);
      if (ks == 0) out[(row0 + h) * D + orow + RS * r] = sL[h] > 0.0f ? acc[r] / sL[h] : 0.0f;
    }
  }
  if (threadIdx.x < GG && lse)
    lse[row0 + threadIdx.x] = sL[threadIdx.x] > 0.0f ? sM[threadIdx.x] + logf(sL[threadIdx.x]) : kNegInf;
}

constexpr int kMfmaThreads = 256;

// POLAR: keys are polar codes (4-bit level-1, 2-bit higher angles, head_dim 128).  With the
// unit vector u = R_p (cos theta_p, sin theta_p) on level-1 pair p (R_p the product of the
// cos / sin factors of p's ancestors), <q_x, u> = sum_p R_p T[p][c_p] for the per-query pair
// table T[p][c] = q_x,2p cos theta_c + q_x,2p+1 sin theta_c (the workgroup builds it for its four
// heads in LDS from q_x).  Lane (token n, K slice kg) forms R_p top-down for its 16 pairs
// [16 kg, 16 kg + 16) and sums R_p T[p][c_p] for all four heads in float32; the four K slices'
// sums meet by two shuffle rounds in the lane of head kg.
template <int BK, bool QJL, bool GATHER, bool LOGITS, bool POLAR = false>
__global__ __launch_bounds__(kMfmaThreads, 3) void decode_mfma_kernel(DecodeArgs A) {
  constexpr int D = 128, G = 4, NW = kMfmaThreads / 64;
  // polar: cos / sin of levels 2..7 [6][4]; the four heads' pair tables [64 pairs][16 codes]
  __shared__ float2 ptab[POLAR ? 6 * 4 : 1];
  __shared__ __attribute__((aligned(16))) float4 ptq[POLAR ? 64 * 16 : 1];
  __shared__ float pqx[POLAR ? G : 1][POLAR ? D : 1];
  // value code -> bf16 (hi, lo) pair of its level / sqrt(d): 16 words in 16 distinct banks, so lookups
  // never conflict (equal codes are broadcast)
  __shared__ uint32_t vtab[16];
  // Value-code staging, rows padded to TS words so that the four K-slices of a write (and the
  // 16 rows of a 16-byte read) fall on distinct LDS banks.  The cross-wave merge reuses it.
  constexpr int TS = 20;
  __shared__ __attribute__((aligned(16))) union {
    uint32_t vst[NW][16 * TS];       // value codes: [coordinate octet][token]
    float red[NW][G][D + 2];         // cross-wave merge
  } sh;
  __shared__ __attribute__((aligned(16))) uint32_t wstage[NW][2][4 * 16];  // [w half][head][token] bf16 in high 16 bits
  __shared__ __attribute__((aligned(16))) uint32_t wzero[4];              // B rows of the unused value columns
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.z, hkv = blockIdx.y, chunk = blockIdx.x;
  const int64_t qrow0 = (int64_t)b * A.q_heads + (int64_t)hkv * G;
  if (A.gate && !(A.gate[qrow0] | A.gate[qrow0 + 1] | A.gate[qrow0 + 2] | A.gate[qrow0 + 3]))
    return;                // no head of the group reads the cold tokens: the merge ignores them

  if (threadIdx.x < 16) vtab[threadIdx.x] = bf16_pair(A.val_levels[threadIdx.x] * A.inv_sqrt_d);
  if (threadIdx.x < 4) wzero[threadIdx.x] = 0u;
  if constexpr (POLAR) {
    if (threadIdx.x < 24) {
      const int l = threadIdx.x >> 2, c = threadIdx.x & 3;      // level 2 + l
      ptab[threadIdx.x] = make_float2(A.pcs[2 * ((1 + l) * 16 + c)], A.pcs[2 * ((1 + l) * 16 + c) + 1]);
    }
    for (int e = threadIdx.x; e < G * D; e += kMfmaThreads) pqx[e / D][e % D] = A.qx[qrow0 * D + e];
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 16; e += kMfmaThreads) {
      const int p = e >> 4, c = e & 15;
      const float ct = A.pcs[2 * c], st = A.pcs[2 * c + 1];   // level-1 angle c
      float4 t;
      t.x = fmaf(pqx[0][2 * p + 1], st, pqx[0][2 * p] * ct);
      t.y = fmaf(pqx[1][2 * p + 1], st, pqx[1][2 * p] * ct);
      t.z = fmaf(pqx[2][2 * p + 1], st, pqx[2][2 * p] * ct);
      t.w = fmaf(pqx[3][2 * p + 1], st, pqx[3][2 * p] * ct);
      ptq[e] = t;
    }
  }

  // key levels as int8 limbs: gamma ~= (256 hi + lo) / F, byte c of each table word = code c
  const float fk = A.key_fix;
  uint32_t th[2] = {0, 0}, tl[2] = {0, 0};
#pragma unroll
  for (int c = 0; c < (1 << BK); ++c) {
    int hi, lo;
    int8_limbs((int)rintf(A.key_levels[c] * fk), hi, lo);
    th[c >> 2] |= (uint32_t)(hi & 0xFF) << (8 * (c & 3));
    tl[c >> 2] |= (uint32_t)(lo & 0xFF) << (8 * (c & 3));
  }

  // Score products with the query operands as A (rows = (head, part), from mfma_prep_kernel)
  // and the 16 tokens' operands as B, so lane (K slice / head kg, column n) ends with every
  // part of head kg for token n: the lane owns score (token n, head kg), and each lane loads
  // only its own token's fields (key group kg, sketch word kg, value quarter kg, norms).
  const int n = lane & 15, kg = lane >> 4;
  constexpr int NCK = POLAR ? 0 : 4;                         // key operand chunks
  i32x4 Aq[POLAR ? 1 : 4], Aj[2];
  float bk16, bk8, bq, oq, kpol;
  {
    const u32x4* bp = reinterpret_cast<const u32x4*>(
        A.bop + (((int64_t)b * A.kv_heads + hkv) * 64 + lane) * (POLAR ? kPolarLaneWords : 32));
    u32x4 w[NCK + 3];
#pragma unroll
    for (int i = 0; i < NCK + 3; ++i) w[i] = bp[i];
    if constexpr (!POLAR) {
#pragma unroll
      for (int j = 0; j < 4; ++j) Aq[j] = __builtin_bit_cast(i32x4, w[j]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) Aj[j] = __builtin_bit_cast(i32x4, w[NCK + j]);
    // logits in base-2 units (exp2(l2 - m2) = exp(logit - m)): the softmax scale, 1 / sqrt(d)
    // and log2(e) ride on the part weights, the QJL coefficient on the sketch's
    const float ks = A.scale * A.inv_sqrt_d * kLog2e, qs = A.scale * A.qjl_coef * kLog2e;
    const float bk = __uint_as_float(w[NCK + 2][0]);
    bk16 = 65536.0f * bk * ks;
    bk8 = 256.0f * bk * ks;
    // polar: the logit is r_k <q_x, u> (u of unit norm) times the scale
    kpol = A.scale * kLog2e;
    bq = __uint_as_float(w[NCK + 2][1]) * qs;
    oq = __uint_as_float(w[NCK + 2][2]) * qs;
  }
  __syncthreads();

  const int n_tok = GATHER ? A.k_sel : (int)min((int64_t)A.seq_lens[b], A.capacity);
  const int c0 = chunk * A.chunk, c1 = min(n_tok, c0 + A.chunk);
  const uint8_t* recs = A.records + ((int64_t)b * A.kv_heads + hkv) * A.capacity * A.rec_bytes;
  const int32_t* sel = GATHER ? A.sel_idx + ((int64_t)b * A.kv_heads + hkv) * A.k_sel : nullptr;
  uint32_t* vst = sh.vst[wave];
  uint32_t* wst = wstage[wave][0];

  // value accumulators: lane (column n = 2 h + w half, K slice kg) holds rows 4 kg + r of
  // coordinate tile mt, i.e. o[h][8 (4 kg + r) + mt] for its w half (columns 8..15 unused)
  f32x4 acc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float mrun = kNegInf;    // running maximum (base-2 units) of head kg, uniform across its 16 lanes
  float mthr = kNegInf;    // mrun + kLazy
  float lsum = 0.0f;       // this lane's share of sum_t p_t for head kg
  const int vh = n >> 1;   // head of this lane's value column (n < 8)
  // B rows of the value product: the w half (n & 1) of head vh for tokens 4 kg .. 4 kg + 3
  const uint32_t* wsrc = n < 8 ? wstage[wave][n & 1] + (vh & 3) * 16 + 4 * kg : wzero;

  struct Fields {
    uint32_t kw[POLAR ? 6 : BK];   // polar: level-1 codes of the lane's subtree (2), upper stream (4)
    uint32_t sw;
    u32x4 vw;
    float nk, nrho, nv;
    bool valid;
  };
  // Addresses are always clamped to a record of this (sequence, head), so every load is
  // unconditional (no memory operation under a branch in the loop).  Byte offsets within the
  // (sequence, head) run fit in 32 bits (the host routes larger caches to the generic kernel).
  const uint32_t rb = (uint32_t)A.rec_bytes;
  const uint32_t kofs = (uint32_t)(kg * 4 * BK), sofs = (uint32_t)(A.kbytes + 4 * kg);
  const uint32_t vofs = (uint32_t)(A.kbytes + A.sbytes + 16 * kg), nofs = (uint32_t)A.norm_off;
  // lane offsets of the fields within a token's record run for the unclamped path
  const uint32_t lrec = (uint32_t)n * rb;
  auto fetch = [&](int base, Fields& f) {
    const int p = base + n;
    uint32_t t = (uint32_t)min(p, c1 - 1);
    f.valid = p < c1;
    if (GATHER) {
      const int ts = sel[t];
      f.valid = f.valid && ts >= 0 && (int64_t)ts < A.capacity;
      t = f.valid ? (uint32_t)ts : 0u;
    }
    const uint32_t o = (uint32_t)__umul24(t, rb);
    if constexpr (POLAR) {
      const u32x2 w1 = *reinterpret_cast<const u32x2*>(recs + (size_t)(o + 8 * kg));
      const u32x4 wu = *reinterpret_cast<const u32x4*>(recs + (size_t)(o + 32));
      f.kw[0] = w1[0];
      f.kw[1] = w1[1];
      f.kw[2] = wu[0];
      f.kw[3] = wu[1];
      f.kw[4] = wu[2];
      f.kw[5] = wu[3];
    } else if constexpr (BK == 3) {
      typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
      const u32x3 w = *reinterpret_cast<const u32x3*>(recs + (size_t)(o + kofs));
      f.kw[0] = w[0];
      f.kw[1] = w[1];
      f.kw[2] = w[2];
    } else {
      const u32x2 w = *reinterpret_cast<const u32x2*>(recs + (size_t)(o + kofs));
      f.kw[0] = w[0];
      f.kw[1] = w[1];
    }
    f.sw = QJL ? *reinterpret_cast<const uint32_t*>(recs + (size_t)(o + sofs)) : 0u;
    f.vw = *reinterpret_cast<const u32x4*>(recs + (size_t)(o + vofs));
    const float* nrm = reinterpret_cast<const float*>(recs + (size_t)(o + nofs));
    f.nk = nrm[0];
    f.nrho = nrm[1];
    f.nv = nrm[2];
  };

  // one 16-token step on fields `cur` (tokens base .. base + 15)
  auto step = [&](const Fields& cur, int base) {

    float l2;
    if constexpr (POLAR) {
      // ---- key scores: sum_p R_p T[p][c_p] over the lane's 16 level-1 pairs, all four heads ----
      const uint32_t u3 = cur.kw[5], u2 = cur.kw[4], uw2 = kg < 2 ? cur.kw[2] : cur.kw[3];
      const float2* csl = ptab + 4;                                    // levels 3..7
      const float2 t7 = csl[16 + ((u3 >> 28) & 3u)];
      const float2 t6 = csl[12 + ((u3 >> (24 + 2 * (kg >> 1))) & 3u)];
      const float sroot = ((kg >> 1) ? t7.y : t7.x) * ((kg & 1) ? t6.y : t6.x);
      const float2 t5 = csl[8 + ((u3 >> (16 + 2 * kg)) & 3u)];
      float s4[2] = {sroot * t5.x, sroot * t5.y}, s3[4], s2[8];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float2 t = csl[4 + ((u3 >> (4 * kg + 2 * i)) & 3u)];
        s3[2 * i] = s4[i] * t.x;
        s3[2 * i + 1] = s4[i] * t.y;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 t = csl[(u2 >> (8 * kg + 2 * i)) & 3u];
        s2[2 * i] = s3[i] * t.x;
        s2[2 * i + 1] = s3[i] * t.y;
      }
      // level-1 codes pre-scaled to float4 offsets within a pair's 16-entry table: byte k of
      // lo / hi = code of pair 2 (4 w + k) / 2 (4 w + k) + 1 times 16 bytes
      const float4* tq = ptq + 256 * kg;                               // pairs 16 kg ..
      float dot[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int wq = 0; wq < 2; ++wq) {
        uint32_t lo = (cur.kw[wq] << 4) & 0xF0F0F0F0u, hi = cur.kw[wq] & 0xF0F0F0F0u;
        asm volatile("" : "+v"(lo));
        asm volatile("" : "+v"(hi));
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
          const int k = 4 * wq + k2;                                   // level-2 node
          const float2 l2 = ptab[(uw2 >> (16 * (kg & 1) + 2 * k)) & 3u];
          const float ra = s2[k] * l2.x, rb = s2[k] * l2.y;
          const uint8_t* tb = reinterpret_cast<const uint8_t*>(tq + 32 * k);
          const float4 ta = *reinterpret_cast<const float4*>(tb + ((lo >> (8 * k2)) & 0xFFu));
          const float4 tc = *reinterpret_cast<const float4*>(tb + 256 + ((hi >> (8 * k2)) & 0xFFu));
          dot[0] = fmaf(rb, tc.x, fmaf(ra, ta.x, dot[0]));
          dot[1] = fmaf(rb, tc.y, fmaf(ra, ta.y, dot[1]));
          dot[2] = fmaf(rb, tc.z, fmaf(ra, ta.z, dot[2]));
          dot[3] = fmaf(rb, tc.w, fmaf(ra, ta.w, dot[3]));
        }
      }
      // the token's four K slices (lanes n + 16 kg') meet in the lane of head kg
      const bool upper = kg >> 1, odd = kg & 1;
      const float b0 = (upper ? dot[2] : dot[0]) + __shfl_xor(upper ? dot[0] : dot[2], 32);
      const float b1 = (upper ? dot[3] : dot[1]) + __shfl_xor(upper ? dot[1] : dot[3], 32);
      const float qu = (odd ? b1 : b0) + __shfl_xor(odd ? b0 : b1, 16);
      i32x4 Cq = i32x4{0, 0, 0, 0};
      if (QJL) {
#pragma unroll
        for (int j = 1; j < 4; j += 2) {
          i32x4 q;
#pragma unroll
          for (int w = 0; w < 4; ++w) q[w] = (int)(cur.sw & (0x01010101u << (2 * (j & 2) + w)));
          Cq = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aj[j >> 1], q, Cq, 0, 0, 0);
        }
      }
      l2 = cur.nk * qu * kpol;
      if (QJL) l2 = fmaf(cur.nrho, fmaf((float)((Cq[0] << 16) + (Cq[1] << 8) + Cq[2]), bq, oq), l2);
    } else {
    // ---- key scores (exact int32), token operands from the level tables ----
    uint32_t sel[8];
    if constexpr (BK == 3) {
      const uint32_t top = group3_top(cur.kw[0], cur.kw[1], cur.kw[2]);
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        sel[2 * t] = cur.kw[t] & 0x07070707u;
        sel[2 * t + 1] = (cur.kw[t] >> 3) & 0x07070707u;
      }
      sel[6] = top & 0x07070707u;
      sel[7] = (top >> 3) & 0x07070707u;
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) sel[t] = (cur.kw[t >> 2] >> (2 * (t & 3))) & 0x03030303u;
    }
    i32x4 C0 = i32x4{0, 0, 0, 0}, Cq = C0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const i32x4 bt = i32x4{(int)__builtin_amdgcn_perm(th[1], th[0], sel[2 * j]),
                             (int)__builtin_amdgcn_perm(th[1], th[0], sel[2 * j + 1]),
                             (int)__builtin_amdgcn_perm(tl[1], tl[0], sel[2 * j]),
                             (int)__builtin_amdgcn_perm(tl[1], tl[0], sel[2 * j + 1])};
      C0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aq[j], bt, C0, 0, 0, 0);
      if (QJL && (j & 1)) {
        i32x4 q;
#pragma unroll
        for (int w = 0; w < 4; ++w) q[w] = (int)(cur.sw & (0x01010101u << (2 * (j & 2) + w)));
        Cq = __builtin_amdgcn_mfma_i32_16x16x64_i8(Aj[j >> 1], q, Cq, 0, 0, 0);
      }
    }
    // parts of head kg for token n: weights 2^24, 2^16, 2^8 (|C0[0]| < 2^21 and |C0[1]| < 2^22,
    // so 256 C0[0] + C0[1] fits in int32); sketch sum 2^16 Cq0 + 2^8 Cq1 + Cq2 < 2^31
    l2 = cur.nk * fmaf((float)((C0[0] << 8) + C0[1]), bk16, (float)C0[2] * bk8);
    if (QJL) l2 = fmaf(cur.nrho, fmaf((float)((Cq[0] << 16) + (Cq[1] << 8) + Cq[2]), bq, oq), l2);
    }
    const float logit = cur.valid ? l2 : kNegInf;
    if (LOGITS && cur.valid) A.logits[(qrow0 + kg) * A.logit_stride + base + n] = logit * kLn2;
    // ---- running maximum per head, shared by its 16 lanes, raised lazily (rare branch) ----
    if (__ballot(logit > mthr) != 0ull) {
      float tmax = logit;
#pragma unroll
      for (int msk = 1; msk < 16; msk <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, msk));
      const bool raise = tmax > mthr;                 // uniform within each head
      const float fct = raise ? (mrun == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mrun - tmax)) : 1.0f;
      lsum *= fct;
      mrun = raise ? tmax : mrun;
      mthr = mrun + kLazy;
      // rescale the value accumulators of head vh by that head's factor
      const float fv = __shfl(fct, 16 * (vh & 3));    // lane 16 h holds head h's factor
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[mt] *= fv;
    }
    // an invalid token's logit is -inf, and mrun is finite once a step has run (its first
    // token is valid), so only a gathered step (invalid indices anywhere) needs the select
    const float p = (GATHER && !cur.valid) ? 0.0f : __builtin_amdgcn_exp2f(logit - mrun);
    lsum += p;
    {
      // w = hi + lo, hi = w truncated to bf16, lo = w - hi; the value products read the top 16
      // bits of each word, so lo is truncated to bf16 as well (w within 2^-14 relative)
      const float w = p * cur.nv;
      wst[kg * 16 + n] = __float_as_uint(w);
      wst[64 + kg * 16 + n] = __float_as_uint(w - __uint_as_float(__float_as_uint(w) & 0xFFFF0000u));
    }
    // this token's value codes, coordinate quarter kg: word r = coordinate octet 4 kg + r
#pragma unroll
    for (int r = 0; r < 4; ++r) vst[(4 * kg + r) * TS + n] = cur.vw[r];
    wave_lds_sync();
    // ---- values: B = w halves of (head vh) for tokens 4 kg .. 4 kg + 3, A = level halves ----
    const u32x4 w4 = *reinterpret_cast<const u32x4*>(wsrc);
    const u32x4 codes = *reinterpret_cast<const u32x4*>(vst + n * TS + 4 * kg);   // row n = coordinate octet
    wave_lds_sync();
    u32x4 bw;
#pragma unroll
    for (int d = 0; d < 4; ++d) bw[d] = __builtin_amdgcn_perm(w4[d], w4[d], 0x03020302u);
    const bf16x8 Bv = __builtin_bit_cast(bf16x8, bw);
    // low / high nibbles of the code bytes, pre-scaled to LDS byte offsets into vtab, so each
    // lookup address is one byte extract
    u32x4 nib[2];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      nib[0][d] = (codes[d] << 2) & 0x3C3C3C3Cu;
      nib[1][d] = (codes[d] >> 2) & 0x3C3C3C3Cu;
      // opaque to the optimizer, which would otherwise fold the scaling back into every
      // extract (shift + mask per lookup instead of one bit-field extract)
      asm volatile("" : "+v"(nib[0][d]));
      asm volatile("" : "+v"(nib[1][d]));
    }
    const uint8_t* vt = reinterpret_cast<const uint8_t*>(vtab);
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {                  // coordinate tiles 2 pr, 2 pr + 1
      u32x4 a0, a1;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        a0[d] = *reinterpret_cast<const uint32_t*>(vt + ((nib[0][d] >> (8 * pr)) & 0xFFu));
        a1[d] = *reinterpret_cast<const uint32_t*>(vt + ((nib[1][d] >> (8 * pr)) & 0xFFu));
      }
      acc[2 * pr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), Bv, acc[2 * pr], 0, 0, 0);
      acc[2 * pr + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), Bv, acc[2 * pr + 1], 0, 0, 0);
    }
  };
  // two-way unrolled so that the prefetched fields alternate between f0 and f1 (no copies)
  Fields f0, f1;
  int base = c0 + wave * 16;
  if (base < c1) fetch(base, f0);
  while (base < c1) {
    fetch(base + NW * 16, f1);       // prefetch the next step's record fields (clamped)
    step(f0, base);
    base += NW * 16;
    if (base >= c1) break;
    fetch(base + NW * 16, f0);
    step(f1, base);
    base += NW * 16;
  }

  // ---- merge: sum the two w halves (columns 2h, 2h+1), the token lanes' l, then the waves ----
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[mt][r] += __shfl_xor(acc[mt][r], 1);
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) lsum += __shfl_xor(lsum, msk);
  __syncthreads();              // every wave is done with the staging area the merge reuses
  float (*red)[G][D + 2] = sh.red;
  if (n == 0) {                 // lane 16 h: head h's m (natural units) and l
    red[wave][kg][0] = mrun * kLn2;
    red[wave][kg][1] = lsum;
  }
  if (n < 8 && (n & 1) == 0) {  // column (h, hi half) lanes: o[h][8 (4 kg + r) + mt]
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][vh][2 + 8 * (4 * kg + r) + mt] = acc[mt][r];
  }
  __syncthreads();
  const int stride = D + 2;
  for (int e = threadIdx.x; e < G * stride; e += blockDim.x) {
    const int hh = e / stride, col = e % stride;
    float mx = kNegInf;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) mx = fmaxf(mx, red[w2][hh][0]);
    float v = mx;
    if (col > 0) {
      v = 0.0f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2)
        if (red[w2][hh][0] != kNegInf) v += red[w2][hh][col] * __expf(red[w2][hh][0] - mx);
    }
    A.part[((qrow0 + hh) * A.n_chunks + chunk) * stride + col] = v;
  }
}

// Merge: log-sum-exp of the chunk partials, the exact (hot) segment in the same softmax
// (Monarch v3 page, "Wie es funktioniert"), and o = Pi^T o_x + o_hot, divided by the sum.
// One output of y = M v (M [rows][D] row-major float32, v float32 in LDS), split over two
// threads (half h of the row each): 64 contiguous floats as independent 16-byte loads (one memory
// round trip), combined with a shuffle.
template <int D>
__device__ __forceinline__ float gemv_row_half_f32(const float* __restrict__ mrow, const float* v, int h) {
  constexpr int H = D / 2;
  const float4* p = reinterpret_cast<const float4*>(mrow + h * H);
  float4 w[H / 4];
#pragma unroll
  for (int j = 0; j < H / 4; ++j) w[j] = p[j];
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < H / 4; ++j) {
    const float* vv = v + h * H + 4 * j;
    acc = fmaf(w[j].x, vv[0], acc);
    acc = fmaf(w[j].y, vv[1], acc);
    acc = fmaf(w[j].z, vv[2], acc);
    acc = fmaf(w[j].w, vv[3], acc);
  }
  return acc + __shfl_xor(acc, 1);
}

// Eight consecutive elements [off, off + 8) as float32 (16-byte aligned for 16-bit types,
// 32-byte aligned for float32).
__device__ __forceinline__ void load8(const void* base, tq_dtype dt, int64_t off, float (&v)[8]) {
  if (dt == TQ_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = dt == TQ_BF16 ? bf16_bits_to_f32(w[i] & 0xffffu) : f16_bits_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = dt == TQ_BF16 ? bf16_bits_to_f32(w[i] >> 16) : f16_bits_to_f32(w[i] >> 16);
    }
  }
}

// sum_c o_c[i] exp(m_c - M) over a row's chunk partials [nch][stride] = (m, l, o[0..]), eight
// chunks' loads in flight at a time (a chunk with m = -inf weighs 0)
__device__ __forceinline__ float merge_chunks(const float* pr, int nch, int stride, int i, float M) {
  float acc = 0.0f;
  int c = 0;
  for (; c + 8 <= nch; c += 8) {
    float mc[8], ov[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      mc[u] = pr[(int64_t)(c + u) * stride];
      ov[u] = pr[(int64_t)(c + u) * stride + 2 + i];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      acc = fmaf(ov[u], (M != kNegInf && mc[u] != kNegInf) ? __expf(mc[u] - M) : 0.0f, acc);
  }
  for (; c < nch; ++c) {
    const float mc = pr[(int64_t)c * stride];
    acc = fmaf(pr[(int64_t)c * stride + 2 + i], (M != kNegInf && mc != kNegInf) ? __expf(mc - M) : 0.0f, acc);
  }
  return acc;
}

struct MergeArgs {
  const float* pi_t;      // Pi transposed
  const float* part;
  const void* q;
  tq_dtype q_dt;
  const void* hot_k;
  const void* hot_v;
  tq_dtype hot_dt;
  const int32_t* hot_lens;
  const int32_t* hot_start;   // ring start of each sequence's hot tokens (NULL: slot t = token t)
  const int32_t* gate;        // [B][Hq] nonzero: the head's cold partials count (NULL: all do)
  int hot_add;                // tokens appended past hot_lens in this step (ring mode)
  int64_t hot_capacity, logit_hot_off, logit_stride;
  uint32_t* promo_w;          // hot/cold step: per-token maximum of the open heads' weights (NULL: none)
  const int32_t* promo_n;     // [B] cold tokens
  int64_t promo_stride;       // cold capacity
  float* out;
  float* lse;
  float* logits;
  int d, G, q_heads, kv_heads, n_chunks;
  float scale;
};

constexpr int kMergeThreads = 256;        // without an exact segment
constexpr int kMergeThreadsHot = 1024;    // with one: more token slots per pass

constexpr int kMergeHotLds = 2048;   // exact-segment logits kept in LDS (beyond: recomputed)

template <int D, int NT>
__global__ __launch_bounds__(NT) void decode_merge_kernel(MergeArgs A) {
  // exact segment layout: LPK lanes per token, each owning 8 consecutive coordinates
  constexpr int LPK = D / 8, TPWK = 64 / LPK, TPB = TPWK * (NT / 64);
  __shared__ float qv[D];
  __shared__ float ox[D];
  __shared__ float ohw[NT / 64][D];
  __shared__ float hlog[kMergeHotLds];
  __shared__ float red[NT];
  __shared__ float oxp[NT];   // per-thread partial sums of the rotated-domain output
  const int hq = blockIdx.x, b = blockIdx.y, hkv = hq / A.G;
  const int64_t row = (int64_t)b * A.q_heads + hq;
  constexpr int stride = D + 2;
  const float* pr = A.part + row * A.n_chunks * stride;
  const int n_chunks = (A.gate && A.gate[row] == 0) ? 0 : A.n_chunks;   // gated: hot tokens only
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // block-wide max / sum: wave shuffles, then one LDS word per wave
  auto block_reduce = [&](float v, bool is_max) {
#pragma unroll
    for (int msk = 32; msk > 0; msk >>= 1) {
      const float o = __shfl_xor(v, msk);
      v = is_max ? fmaxf(v, o) : v + o;
    }
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
    for (int w2 = 1; w2 < NT / 64; ++w2) v = is_max ? fmaxf(v, red[w2]) : v + red[w2];
    __syncthreads();
    return v;
  };
  for (int i = threadIdx.x; i < D; i += blockDim.x) qv[i] = load_elem(A.q, A.q_dt, row * D + i);
  // global max over chunk partials and hot logits
  float mx = kNegInf;
  for (int c = threadIdx.x; c < n_chunks; c += blockDim.x) mx = fmaxf(mx, pr[(int64_t)c * stride]);
  const int nh = A.hot_lens ? (int)min((int64_t)A.hot_lens[b] + A.hot_add, A.hot_capacity) : 0;
  const int64_t hs0 = A.hot_start ? A.hot_start[b] : 0;
  // ring slot of hot token t
  auto hslot = [&](int t) -> int64_t {
    const int64_t s = hs0 + t;
    return s >= A.hot_capacity ? s - A.hot_capacity : s;
  };
  const int64_t hbase = ((int64_t)b * A.kv_heads + hkv) * A.hot_capacity * D;
  const int sub = lane % LPK, slot = wave * TPWK + lane / LPK;
  __syncthreads();
  float q8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q8[i] = qv[8 * sub + i];
  // logit of hot token t: the LPK lanes of its slot each take 8 coordinates, then a shuffle sum
  auto hot_logit = [&](int t) {
    float kv[8];
    load8(A.hot_k, A.hot_dt, hbase + hslot(min(t, nh - 1)) * D + 8 * sub, kv);
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) dot = fmaf(q8[i], kv[i], dot);
#pragma unroll
    for (int msk = 1; msk < LPK; msk <<= 1) dot += __shfl_xor(dot, msk);
    return A.scale * dot;
  };
  for (int t0 = 0; t0 < nh; t0 += TPB) {
    const int t = t0 + slot;
    const float lg = hot_logit(t);
    if (t < nh) {
      mx = fmaxf(mx, lg);
      if (sub == 0) {
        if (t < kMergeHotLds) hlog[t] = lg;
        if (A.logits) A.logits[row * A.logit_stride + A.logit_hot_off + t] = lg;
      }
    }
  }
  const float M = block_reduce(mx, true);   // (its barriers also order the hlog writes)
  // sum of weights and the cold rotated-domain output (loads unconditional, weight 0 for an
  // empty chunk, whose partial holds zeros)
  float l = 0.0f;
  for (int c = threadIdx.x; c < n_chunks; c += blockDim.x) {
    const float mc = pr[(int64_t)c * stride];
    l += (M != kNegInf && mc != kNegInf) ? pr[(int64_t)c * stride + 1] * __expf(mc - M) : 0.0f;
  }
  {
    // NT / D threads per coordinate, each over every (NT / D)-th chunk (eight loads in flight),
    // then the NT / D partial sums of a coordinate added in LDS: the chunk count (up to a few
    // hundred for short-chunk scans) no longer sets the number of dependent memory round trips
    constexpr int SPLIT = NT / D;
    const int ci = threadIdx.x % D, sp = threadIdx.x / D;
    float acc = 0.0f;
    int c = sp;
    for (; c + 7 * SPLIT < n_chunks; c += 8 * SPLIT) {
      float mc[8], ov[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        mc[u] = pr[(int64_t)(c + u * SPLIT) * stride];
        ov[u] = pr[(int64_t)(c + u * SPLIT) * stride + 2 + ci];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        acc = fmaf(ov[u], (M != kNegInf && mc[u] != kNegInf) ? __expf(mc[u] - M) : 0.0f, acc);
    }
    for (; c < n_chunks; c += SPLIT) {
      const float mc = pr[(int64_t)c * stride];
      acc = fmaf(pr[(int64_t)c * stride + 2 + ci], (M != kNegInf && mc != kNegInf) ? __expf(mc - M) : 0.0f, acc);
    }
    oxp[sp * D + ci] = acc;
  }
  // hot values: each lane accumulates its 8 coordinates over the tokens of its slot
  float oh8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oh8[i] = 0.0f;
  for (int t0 = 0; t0 < nh; t0 += TPB) {
    const int t = t0 + slot;
    float lg;
    if (t0 + TPB <= kMergeHotLds) lg = hlog[min(t, kMergeHotLds - 1)];
    else lg = hot_logit(t);
    const float p = t < nh ? __expf(lg - M) : 0.0f;
    if (sub == 0) l += p;
    float vv[8];
    load8(A.hot_v, A.hot_dt, hbase + hslot(min(t, nh - 1)) * D + 8 * sub, vv);
#pragma unroll
    for (int i = 0; i < 8; ++i) oh8[i] = fmaf(p, vv[i], oh8[i]);
  }
  // reduce over the token slots of the wave (lanes with the same sub), then over the waves
#pragma unroll
  for (int msk = LPK; msk < 64; msk <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) oh8[i] += __shfl_xor(oh8[i], msk);
  if (lane < LPK) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ohw[wave][8 * sub + i] = oh8[i];
  }
  const float L = block_reduce(l, false);   // (its barriers also order the oxp / oh writes)
  for (int i = threadIdx.x; i < D; i += NT) {
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < NT / D; ++q) v += oxp[q * D + i];
    ox[i] = v;
  }
  __syncthreads();
  // o = Pi^T o_x: output i = row i of the transposed rotation against o_x
  {
    const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
    for (int i0 = 0; i0 < D; i0 += NT / 2) {
      const int i = i0 + r;
      const float o = gemv_row_half_f32<D>(A.pi_t + (int64_t)min(i, D - 1) * D, ox, h);
      if (h == 0 && i < D) {
        float hsum = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < NT / 64; ++w2) hsum += ohw[w2][i];
        A.out[row * D + i] = L > 0.0f ? (o + hsum) / L : 0.0f;
      }
    }
  }
  const float lse_r = L > 0.0f ? M + logf(L) : kNegInf;
  if (threadIdx.x == 0 && A.lse) A.lse[row] = lse_r;
  // hot/cold step: this head's weight exp(logit - lse) of every cold token, folded into the
  // per-token maximum over the open heads (non-negative floats order as their bits)
  if (A.promo_w && A.logits && n_chunks > 0) {
    const int nc = (int)min((int64_t)A.promo_n[b], A.promo_stride);
    const float* lg = A.logits + row * A.logit_stride;
    uint32_t* pw = A.promo_w + (int64_t)b * A.promo_stride;
    for (int t = threadIdx.x; t < nc; t += NT) atomicMax(pw + t, __float_as_uint(__expf(lg[t] - lse_r)));
  }
}

// The merge for every other head_dim (d read at run time, up to 256): one workgroup per query
// row.  Pass 1 takes the maximum over the chunk partials and the exact tokens' logits (one
// thread per token, a plain dot product over d); pass 2 takes the exact tokens 2,048 at a
// time - their weights into LDS, then one thread per coordinate sums weight x value - beside
// the chunk partials, and o = Pi^T o_x + the exact part, over the total weight.
__global__ __launch_bounds__(256) void decode_merge_generic_kernel(MergeArgs A) {
  constexpr int NT = 256;
  __shared__ float qv[kGenMaxD], ox[kGenMaxD], oh[kGenMaxD];
  __shared__ float hp[kMergeHotLds];
  __shared__ float red[NT / 64];
  const int hq = blockIdx.x, b = blockIdx.y, hkv = hq / A.G, d = A.d, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t row = (int64_t)b * A.q_heads + hq;
  const int stride = d + 2;
  const float* pr = A.part + row * A.n_chunks * stride;
  const int n_chunks = (A.gate && A.gate[row] == 0) ? 0 : A.n_chunks;
  auto block_reduce = [&](float v, bool is_max) {
#pragma unroll
    for (int msk = 32; msk > 0; msk >>= 1) {
      const float o = __shfl_xor(v, msk);
      v = is_max ? fmaxf(v, o) : v + o;
    }
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
    for (int w2 = 1; w2 < NT / 64; ++w2) v = is_max ? fmaxf(v, red[w2]) : v + red[w2];
    __syncthreads();
    return v;
  };
  for (int i = tid; i < d; i += NT) {
    qv[i] = load_elem(A.q, A.q_dt, row * d + i);
    oh[i] = 0.0f;
  }
  const int nh = A.hot_lens ? (int)min((int64_t)A.hot_lens[b] + A.hot_add, A.hot_capacity) : 0;
  const int64_t hs0 = A.hot_start ? A.hot_start[b] : 0;
  auto hslot = [&](int t) -> int64_t {
    const int64_t sl = hs0 + t;
    return sl >= A.hot_capacity ? sl - A.hot_capacity : sl;
  };
  const int64_t hbase = ((int64_t)b * A.kv_heads + hkv) * A.hot_capacity * d;
  __syncthreads();
  auto hot_logit = [&](int t) {
    const int64_t o = hbase + hslot(t) * d;
    float dot = 0.0f;
    for (int i = 0; i < d; ++i) dot = fmaf(qv[i], load_elem(A.hot_k, A.hot_dt, o + i), dot);
    return A.scale * dot;
  };
  float mx = kNegInf;
  for (int c = tid; c < n_chunks; c += NT) mx = fmaxf(mx, pr[(int64_t)c * stride]);
  for (int t = tid; t < nh; t += NT) {
    const float lgt = hot_logit(t);
    mx = fmaxf(mx, lgt);
    if (A.logits) A.logits[row * A.logit_stride + A.logit_hot_off + t] = lgt;
  }
  const float M = block_reduce(mx, true);
  float l = 0.0f;
  for (int c = tid; c < n_chunks; c += NT) {
    const float mc = pr[(int64_t)c * stride];
    l += (M != kNegInf && mc != kNegInf) ? pr[(int64_t)c * stride + 1] * __expf(mc - M) : 0.0f;
  }
  {
    // coordinates 32 at a time, 8 threads per coordinate over every 8th chunk, summed in LDS
    const int ci = tid & 31, sp = tid >> 5;
    for (int i0 = 0; i0 < d; i0 += 32) {
      const int i = min(i0 + ci, d - 1);
      float acc = 0.0f;
      for (int c = sp; c < n_chunks; c += NT / 32) {
        const float mc = pr[(int64_t)c * stride];
        acc = fmaf(pr[(int64_t)c * stride + 2 + i], (M != kNegInf && mc != kNegInf) ? __expf(mc - M) : 0.0f, acc);
      }
      hp[sp * 32 + ci] = acc;
      __syncthreads();
      if (tid < 32 && i0 + tid < d) {
        float v = 0.0f;
        for (int q = 0; q < NT / 32; ++q) v += hp[q * 32 + tid];
        ox[i0 + tid] = v;
      }
      __syncthreads();
    }
  }
  for (int t0 = 0; t0 < nh; t0 += kMergeHotLds) {
    const int nb = min(kMergeHotLds, nh - t0);
    for (int t = tid; t < nb; t += NT) {
      const float p = __expf(hot_logit(t0 + t) - M);
      hp[t] = p;
      l += p;
    }
    __syncthreads();
    for (int i = tid; i < d; i += NT) {
      float acc = oh[i];
      for (int t = 0; t < nb; ++t) acc = fmaf(hp[t], load_elem(A.hot_v, A.hot_dt, hbase + hslot(t0 + t) * d + i), acc);
      oh[i] = acc;
    }
    __syncthreads();
  }
  const float L = block_reduce(l, false);
  for (int j = tid; j < d; j += NT) {
    const float* pt = A.pi_t + (int64_t)j * d;
    float o = 0.0f;
    for (int i = 0; i < d; ++i) o = fmaf(pt[i], ox[i], o);
    A.out[row * d + j] = L > 0.0f ? (o + oh[j]) / L : 0.0f;
  }
  if (tid == 0 && A.lse) A.lse[row] = L > 0.0f ? M + logf(L) : kNegInf;
}

template <int D, int GG>
__global__ __launch_bounds__(256) void decode_merge_group_kernel(MergeArgs A) {
  merge_group<D, GG>(A.pi_t, A.part, A.out, A.lse,
                     (int64_t)blockIdx.y * A.q_heads + (int64_t)blockIdx.x * GG, A.n_chunks);
}

static bool mfma_path(const Consts& c, int G) {
  return c.d == 128 && G == 4 && c.vb == 4 && (c.kb == 2 || c.kb == 3) && (c.m == 0 || c.m == 128);
}

// polar keys on the matrix-core path: the shape of the llama8b polar workload
static bool polar_mfma_path(const Consts& c, int G) {
  return c.d == 128 && G == 4 && c.vb == 4 && c.pb1 == 4 && c.pbh == 2 && (c.m == 0 || c.m == 128);
}

bool plan_decode(const Consts& c, int batch, int q_heads, int kv_heads, int64_t n_max,
                 DecodePlan* plan) {
  const int G = q_heads / kv_heads;
  plan->generic = c.d != 64 && c.d != 128;
  if (plan->generic) {
    // every other head_dim: the generic direct kernel, chunks of kDecGenTok tokens
    if (c.polar || G > kSmallMaxG || c.d > kGenMaxD || c.m > kDecGenMaxM || c.rec_bytes > kDecGenMaxRec) return false;
    plan->mfma = false;
    plan->small = false;
    plan->group = G;
    plan->hpl = 1;
    plan->key_pairs = false;
    plan->sign_bytes = false;
    plan->chunk = kDecGenTok;
    plan->lds_bytes = 0;
    plan->n_chunks = (int)std::max<int64_t>(1, (n_max + kDecGenTok - 1) / kDecGenTok);
    const size_t rows = (size_t)std::max(batch, 1) * q_heads;
    plan->ws_qx = 0;
    plan->ws_qs = align256(rows * c.d * 4);
    plan->ws_part = plan->ws_qs + align256(rows * std::max(c.m, 1) * 4);
    plan->ws_bop = plan->ws_part + align256(rows * plan->n_chunks * (c.d + 2) * 4);
    plan->ws_total = plan->ws_bop;
    return true;
  }
  plan->mfma = c.polar ? polar_mfma_path(c, G) : mfma_path(c, G);
  const int hpl = (G % 4 == 0) ? 4 : 1;
  const int lpt = (c.d / 32) * (G / hpl);
  if (lpt > 64 || (lpt & (lpt - 1)) != 0) return false;
  plan->group = G;
  plan->hpl = hpl;
  plan->key_pairs = c.kb <= 3;
  // short caches off the matrix-core path with 4+ query heads per KV head (whose per-query
  // tables cost the most to build): the direct kernel, chunks of 8 .. 64 tokens aiming at ~2
  // workgroups per CU
  plan->small = !c.polar && !plan->mfma && n_max <= kSmallMaxN && G >= 4 && G <= kSmallMaxG && c.m <= kSmallMaxM &&
                c.m % 32 == 0 &&
                (c.d == 64 || c.d == 128);
  // split-K: aim at ~2 blocks per CU (3 on the matrix-core path, whose 256-thread blocks fit
  // three to a CU); chunks of at least 64 tokens
  const int64_t units = (int64_t)std::max(batch, 1) * kv_heads;
  const int64_t target_blocks = (plan->mfma ? 3 : 2) * (int64_t)num_cus();
  int64_t chunk = (n_max * units + target_blocks - 1) / std::max<int64_t>(target_blocks, 1);
  chunk = std::max<int64_t>(chunk, 64);
  chunk = std::min<int64_t>(chunk, 16384);
  chunk = (chunk + 63) / 64 * 64;
  if (plan->small) {
    const int64_t want = (n_max * units + 2 * num_cus() - 1) / (2 * (int64_t)num_cus());
    chunk = 8;
    while (chunk < want && chunk < kSmallMaxTok) chunk *= 2;
  }
  plan->chunk = (int)chunk;
  const size_t key_tab = c.polar ? (size_t)G * (c.d / 2) * 16 + (size_t)(c.plevels - 1) * 32
                                 : (size_t)G * (plan->key_pairs ? (c.d / 2) * (1 << (2 * c.kb)) : c.d * (1 << c.kb));
  const size_t sign_bytes_tab = (size_t)G * (c.m / 8) * 256;
  const size_t sign_nib_tab = (size_t)G * (c.m / 4) * 16;
  const size_t budget = 150 * 1024 / 4;
  // byte-indexed sign tables halve the lookups but cost 8x the table build: only for chunks
  // long enough to amortise it
  plan->sign_bytes = chunk >= 2048 && key_tab + sign_bytes_tab + kMaxLevels <= budget;
  const size_t lut = key_tab + (plan->sign_bytes ? sign_bytes_tab : sign_nib_tab) + kMaxLevels;
  const size_t red = (size_t)kDecodeThreads * 36 + 64;
  const size_t floats = std::max(lut, red);
  if (floats > 160 * 1024 / 4) return false;
  plan->lds_bytes = floats * 4;
  plan->n_chunks = (int)std::max<int64_t>(1, (n_max + chunk - 1) / chunk);
  const size_t rows = (size_t)std::max(batch, 1) * q_heads;
  plan->ws_qx = 0;
  plan->ws_qs = align256(rows * c.d * 4);
  plan->ws_part = plan->ws_qs + align256(rows * std::max(c.m, 1) * 4);
  plan->ws_bop = plan->ws_part + align256(rows * plan->n_chunks * (c.d + 2) * 4);
  plan->ws_total = plan->ws_bop + (plan->mfma ? (size_t)std::max(batch, 1) * kv_heads * 64 *
                                                    (c.polar ? kPolarLaneWords : 32) * 4 : 0);
  return true;
}

static void launch_mfma_prep(const Consts& c, const DevConsts& dc, const void* q, tq_dtype q_dt,
                             int batch, int q_heads, int kv_heads, uint32_t* bop, float* qx, hipStream_t st) {
  const dim3 grid((unsigned)(batch * kv_heads)), hgrid((unsigned)(batch * kv_heads * 4));
  const bool qjl = c.m > 0;
  if (c.polar && qjl)
    hipLaunchKernelGGL((mfma_prep_kernel<2, true, false, true>), grid, dim3(kPrepThreads), 0, st, dc.pi, dc.s_pi, q, q_dt, q_heads, kv_heads, c.key_fix, bop, qx);
  else if (c.polar)
    hipLaunchKernelGGL((mfma_prep_kernel<2, false, false, true>), grid, dim3(kPrepThreads), 0, st, dc.pi, dc.s_pi, q, q_dt, q_heads, kv_heads, c.key_fix, bop, qx);
  else if (c.kb == 3 && qjl)
    hipLaunchKernelGGL((mfma_prep_head_kernel<3, true>), hgrid, dim3(kPrepThreads), 0, st, dc.pi, dc.s_pi, q, q_dt, q_heads, kv_heads, c.key_fix, bop);
  else if (c.kb == 3)
    hipLaunchKernelGGL((mfma_prep_head_kernel<3, false>), hgrid, dim3(kPrepThreads), 0, st, dc.pi, dc.s_pi, q, q_dt, q_heads, kv_heads, c.key_fix, bop);
  else if (qjl)
    hipLaunchKernelGGL((mfma_prep_head_kernel<2, true>), hgrid, dim3(kPrepThreads), 0, st, dc.pi, dc.s_pi, q, q_dt, q_heads, kv_heads, c.key_fix, bop);
  else
    hipLaunchKernelGGL((mfma_prep_head_kernel<2, false>), hgrid, dim3(kPrepThreads), 0, st, dc.pi, dc.s_pi, q, q_dt, q_heads, kv_heads, c.key_fix, bop);
}

template <int BK, bool QJL, bool POLAR = false>
static void launch_mfma_bk(const DecodeArgs& a, bool gather, bool logits, dim3 grid, hipStream_t st) {
  if (gather && logits)
    hipLaunchKernelGGL((decode_mfma_kernel<BK, QJL, true, true, POLAR>), grid, dim3(kMfmaThreads), 0, st, a);
  else if (gather)
    hipLaunchKernelGGL((decode_mfma_kernel<BK, QJL, true, false, POLAR>), grid, dim3(kMfmaThreads), 0, st, a);
  else if (logits)
    hipLaunchKernelGGL((decode_mfma_kernel<BK, QJL, false, true, POLAR>), grid, dim3(kMfmaThreads), 0, st, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<BK, QJL, false, false, POLAR>), grid, dim3(kMfmaThreads), 0, st, a);
}

static void launch_mfma_scan(const DecodeArgs& a, int kb, bool qjl, bool gather, bool logits, dim3 grid,
                             hipStream_t st, bool polar = false) {
  if (polar && qjl) launch_mfma_bk<2, true, true>(a, gather, logits, grid, st);
  else if (polar) launch_mfma_bk<2, false, true>(a, gather, logits, grid, st);
  else if (kb == 3 && qjl) launch_mfma_bk<3, true>(a, gather, logits, grid, st);
  else if (kb == 3) launch_mfma_bk<3, false>(a, gather, logits, grid, st);
  else if (qjl) launch_mfma_bk<2, true>(a, gather, logits, grid, st);
  else launch_mfma_bk<2, false>(a, gather, logits, grid, st);
}

template <int HPL>
static void launch_scan_hpl(const DecodeArgs& a, int kb, int vb, bool polar, dim3 grid, size_t lds,
                            hipStream_t st) {
  if (polar) {
#define TQ_DECP(BV_)                                                                             \
    if (vb == BV_) {                                                                             \
      allow_lds(decode_scan_kernel<HPL, 4, BV_, true>, lds);                                      \
      hipLaunchKernelGGL((decode_scan_kernel<HPL, 4, BV_, true>), grid, dim3(kDecodeThreads), lds, st, a); \
      return;                                                                                    \
    }
    TQ_DECP(1) TQ_DECP(2) TQ_DECP(3) TQ_DECP(4)
#undef TQ_DECP
    return;
  }
#define TQ_DEC(BK_, BV_)                                                                         \
  if (kb == BK_ && vb == BV_) {                                                                  \
    allow_lds(decode_scan_kernel<HPL, BK_, BV_>, lds);                                            \
    hipLaunchKernelGGL((decode_scan_kernel<HPL, BK_, BV_>), grid, dim3(kDecodeThreads), lds, st, a); \
    return;                                                                                      \
  }
  TQ_DEC(1, 1) TQ_DEC(1, 2) TQ_DEC(1, 3) TQ_DEC(1, 4) TQ_DEC(2, 1) TQ_DEC(3, 1) TQ_DEC(4, 1)
  TQ_DEC(2, 2) TQ_DEC(2, 3) TQ_DEC(2, 4) TQ_DEC(3, 2) TQ_DEC(3, 3) TQ_DEC(3, 4)
  TQ_DEC(4, 2) TQ_DEC(4, 3) TQ_DEC(4, 4)
#undef TQ_DEC
}

static hipError_t launch_merge(const Consts& c, const MergeArgs& mg, int batch, hipStream_t stream);

hipError_t launch_decode(const Consts& c, const DevConsts& dc, const DecodePlan& plan, const void* q,
                         tq_dtype q_dt, int batch, int q_heads, int kv_heads, const void* records,
                         int64_t capacity, const int32_t* seq_lens, const void* hot_k,
                         const void* hot_v, tq_dtype hot_dt, const int32_t* hot_lens,
                         int64_t hot_capacity, const int32_t* sel_idx, int k_sel, float scale,
                         float* out, float* lse, float* logits, void* workspace,
                         hipStream_t stream, const ProfileEvents& ev, const DecodeHooks* hooks) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* qx = reinterpret_cast<float*>(ws + plan.ws_qx);
  float* qs = reinterpret_cast<float*>(ws + plan.ws_qs);
  float* part = reinterpret_cast<float*>(ws + plan.ws_part);
  const float sc = scale > 0.0f ? scale : c.inv_sqrt_d;
  const int rows = batch * q_heads;
  uint32_t* bop = reinterpret_cast<uint32_t*>(ws + plan.ws_bop);
  // the matrix-core kernel addresses a (sequence, head) run with 32-bit byte offsets
  const bool mfma = plan.mfma && capacity < (int64_t(1) << 24) &&
                    capacity * (int64_t)c.rec_bytes < (int64_t(1) << 31);
  if (mfma)
    launch_mfma_prep(c, dc, q, q_dt, batch, q_heads, kv_heads, bop, qx, stream);
  else
    hipLaunchKernelGGL(query_prep_kernel, dim3(rows), dim3(kQueryPrepThreads), 0, stream, dc.pi, dc.s, c.d, c.m, q,
                       q_dt, qx, qs);
  const int64_t n_cold = sel_idx ? k_sel : capacity;
  const int64_t lstride = n_cold + (hot_lens ? hot_capacity : 0);
  DecodeArgs a;
  a.qx = qx;
  a.qs = qs;
  a.bop = bop;
  a.records = static_cast<const uint8_t*>(records);
  a.seq_lens = seq_lens;
  a.sel_idx = sel_idx;
  a.gate = hooks ? hooks->gate : nullptr;
  a.part = part;
  a.logits = logits;
  a.capacity = capacity;
  a.logit_stride = lstride;
  a.d = c.d;
  a.m = c.m;
  a.kbytes = c.kbytes;
  a.sbytes = c.sbytes;
  a.rec_bytes = c.rec_bytes;
  a.norm_off = c.norm_off;
  a.kb = c.kb;
  a.vb = c.vb;
  a.G = plan.group;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.k_sel = k_sel;
  a.chunk = plan.chunk;
  a.n_chunks = plan.n_chunks;
  a.sign_bytes = plan.sign_bytes ? 1 : 0;
  a.scale = sc;
  a.inv_sqrt_d = c.inv_sqrt_d;
  a.qjl_coef = c.qjl_coef;
  a.key_fix = c.key_fix;
  for (int i = 0; i < kMaxLevels; ++i) {
    a.key_levels[i] = c.key_levels[i];
    a.val_levels[i] = c.val_levels[i];
  }
  a.pcs = dc.polar.cs32;
  a.pb1 = c.pb1;
  a.pbh = c.pbh;
  a.plevels = c.plevels;
  a.l1_bytes = c.l1_bytes;
  dim3 grid(plan.n_chunks, kv_heads, batch);
  ev.before(stream);
  if (plan.generic) {
    hipLaunchKernelGGL(decode_generic_kernel, grid, dim3(kSmallThreads), 0, stream, a);
  } else if (mfma) {
    launch_mfma_scan(a, c.kb, c.m > 0, sel_idx != nullptr, logits != nullptr, grid, stream, c.polar != 0);
  } else if (plan.small) {
    if (c.d == 128) launch_small_d<128>(a, c.kb, c.vb, grid, stream);
    else launch_small_d<64>(a, c.kb, c.vb, grid, stream);
  } else if (plan.hpl == 4) {
    launch_scan_hpl<4>(a, c.kb, c.vb, c.polar != 0, grid, plan.lds_bytes, stream);
  } else {
    launch_scan_hpl<1>(a, c.kb, c.vb, c.polar != 0, grid, plan.lds_bytes, stream);
  }
  ev.after(stream);
  MergeArgs mg;
  mg.pi_t = dc.pi_t;
  mg.part = part;
  mg.q = q;
  mg.q_dt = q_dt;
  mg.hot_k = hot_k;
  mg.hot_v = hot_v;
  mg.hot_dt = hot_dt;
  mg.hot_lens = hot_lens;
  mg.hot_start = hooks ? hooks->hot_start : nullptr;
  mg.gate = hooks ? hooks->gate : nullptr;
  mg.hot_add = hooks ? hooks->hot_add : 0;
  mg.promo_w = hooks ? hooks->promo_w : nullptr;
  mg.promo_n = seq_lens;
  mg.promo_stride = capacity;
  mg.hot_capacity = hot_capacity;
  mg.logit_hot_off = n_cold;
  mg.logit_stride = lstride;
  mg.out = out;
  mg.lse = lse;
  mg.logits = logits;
  mg.d = c.d;
  mg.G = plan.group;
  mg.q_heads = q_heads;
  mg.kv_heads = kv_heads;
  mg.n_chunks = plan.n_chunks;
  mg.scale = sc;
  return launch_merge(c, mg, batch, stream);
}

// The merge of chunk partials (and the exact segment, if any) into out / lse.
static hipError_t launch_merge(const Consts& c, const MergeArgs& mg, int batch, hipStream_t stream) {
  const int q_heads = mg.q_heads, kv_heads = mg.kv_heads;
  // the hot/cold step's promotion weights are folded in by the merge with an exact segment
  if (mg.promo_w && (!mg.hot_lens || (c.d != 64 && c.d != 128))) return hipErrorInvalidValue;
  const dim3 mgrid(q_heads, batch);
  if (c.d != 64 && c.d != 128) {
    hipLaunchKernelGGL(decode_merge_generic_kernel, mgrid, dim3(256), 0, stream, mg);
  } else if (mg.hot_lens) {
    if (c.d == 128) hipLaunchKernelGGL((decode_merge_kernel<128, kMergeThreadsHot>), mgrid, dim3(kMergeThreadsHot), 0, stream, mg);
    else hipLaunchKernelGGL((decode_merge_kernel<64, kMergeThreadsHot>), mgrid, dim3(kMergeThreadsHot), 0, stream, mg);
  } else if (mg.G == 4 || mg.G == 2) {
    // one block per query head: more blocks, each with a quarter (half) of the group's work
    if (c.d == 128) hipLaunchKernelGGL((decode_merge_group_kernel<128, 1>), mgrid, dim3(256), 0, stream, mg);
    else hipLaunchKernelGGL((decode_merge_group_kernel<64, 1>), mgrid, dim3(256), 0, stream, mg);
  } else if (mg.G == 1 && !mg.gate && mg.n_chunks <= 16 * 256 / c.d) {
    // one query head per KV head: the per-head merge, chunk partials split over the block
    if (c.d == 128) hipLaunchKernelGGL((decode_merge_group_kernel<128, 1>), mgrid, dim3(256), 0, stream, mg);
    else hipLaunchKernelGGL((decode_merge_group_kernel<64, 1>), mgrid, dim3(256), 0, stream, mg);
  } else {
    if (c.d == 128) hipLaunchKernelGGL((decode_merge_kernel<128, kMergeThreads>), mgrid, dim3(kMergeThreads), 0, stream, mg);
    else hipLaunchKernelGGL((decode_merge_kernel<64, kMergeThreads>), mgrid, dim3(kMergeThreads), 0, stream, mg);
  }
  return hipGetLastError();
}

// =========================================================================================
// Self-Indexing sign index (Self-Indexing KVCache page, "Methodologie" 1-2): per (sequence,
// KV head) the channel mean mu over the tokens indexed, bit = [k >= mu] (float32), one 4-bit
// pattern per 4-channel group, and 16 centroids per group = mean of the members' (k - mu)
// sub-vectors (0 for a pattern without members).  Sums are float64 and taken in a fixed
// order (per-chunk partial sums, then chunks in order), so the result is deterministic.
// =========================================================================================
constexpr int kIndexSub = 64;    // tokens staged per sub-tile in the pattern / centroid pass

IndexPlan plan_index(const Consts& c, int batch, int heads, int64_t n_tokens) {
  IndexPlan p;
  int64_t chunk = 4096;
  const int64_t max_chunks = 64;
  if (n_tokens > chunk * max_chunks) chunk = (n_tokens + max_chunks - 1) / max_chunks;
  chunk = (chunk + kIndexSub - 1) / kIndexSub * kIndexSub;
  p.chunk = (int)chunk;
  p.n_chunks = (int)std::max<int64_t>(1, (n_tokens + chunk - 1) / chunk);
  const size_t units = (size_t)std::max(batch, 1) * heads;
  const int ng = c.d / 4;
  p.ws_mean = 0;                                                         // f64 [units][chunks][d], then f32 mu [units][d]
  const size_t mean_bytes = align256(units * p.n_chunks * c.d * 8) + align256(units * c.d * 4);
  p.ws_csum = mean_bytes;                                                // f64 [units][chunks][ng][16][4]
  p.ws_ccnt = p.ws_csum + align256(units * p.n_chunks * ng * 16 * 4 * 8);  // i32 [units][chunks][ng][16]
  p.ws_total = p.ws_ccnt + align256(units * p.n_chunks * ng * 16 * 4);
  return p;
}

struct IndexArgs {
  const void* k;
  tq_dtype dt;
  int d, heads, chunk, n_chunks;
  int64_t n_tokens, seq_stride, tok_stride, head_stride, capacity, first_slot;
  double* mean_part;
  float* mu;
  double* csum;
  int32_t* ccnt;
  uint8_t* index;
  float* codebook;
  float* mean_out;
};

// Eight consecutive elements of a key row as raw words (16-bit types: 4 words, float32: 8),
// converted later, so that a load can stay in flight across other work.
template <tq_dtype DT>
__device__ __forceinline__ void load8_raw(const void* base, int64_t off, uint32_t (&r)[8]) {
  if constexpr (DT == TQ_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + off);
    const uint4 a = p[0], b = p[1];
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w; r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  }
}
template <tq_dtype DT>
__device__ __forceinline__ void cvt8(const uint32_t (&r)[8], float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (DT == TQ_F32) v[i] = __uint_as_float(r[i]);
    else {
      const uint32_t h = (i & 1) ? r[i / 2] >> 16 : r[i / 2] & 0xFFFFu;
      v[i] = DT == TQ_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
    }
  }
}

// Per-chunk channel sums of the keys.  Thread (token lane tl, channel octet cg) sums channels
// 8 cg .. 8 cg + 7 of tokens t0 + tl, t0 + tl + L, ... in order (16-byte loads; the host checks
// that base and strides are 16-byte aligned); the L lanes' sums are then added in lane order.
template <tq_dtype DT>
__global__ __launch_bounds__(256) void index_mean_kernel(IndexArgs A) {
  __shared__ double part[256 * 8];
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, d = A.d;
  const int ncg = d / 8, L = 256 / ncg;
  const int cg = threadIdx.x % ncg, tl = threadIdx.x / ncg;
  const int64_t t0 = (int64_t)chunk * A.chunk, t1 = min(A.n_tokens, t0 + A.chunk);
  const int64_t base = (int64_t)b * A.seq_stride + (int64_t)h * A.head_stride + 8 * cg;
  double s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.0;
  // four rows in flight per round (clamped loads; rows past t1 are not added)
  for (int64_t t = t0 + tl; t < t1; t += 4 * L) {
    uint32_t raw[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8_raw<DT>(A.k, base + min(t + u * L, t1 - 1) * A.tok_stride, raw[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float v[8];
      cvt8<DT>(raw[u], v);
      if (t + u * L < t1)
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] += (double)v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[threadIdx.x * 8 + i] = s[i];
  __syncthreads();
  if (tl == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double tot = 0.0;
      for (int u = 0; u < L; ++u) tot += part[(u * ncg + cg) * 8 + i];
      A.mean_part[(((int64_t)b * A.heads + h) * A.n_chunks + chunk) * d + 8 * cg + i] = tot;
    }
  }
}

__global__ void index_mean_final_kernel(IndexArgs A) {
  const int h = blockIdx.x, b = blockIdx.y, d = A.d;
  const int64_t unit = (int64_t)b * A.heads + h;
  for (int ch = threadIdx.x; ch < d; ch += blockDim.x) {
    double s = 0.0;
    for (int c = 0; c < A.n_chunks; ++c) s += A.mean_part[(unit * A.n_chunks + c) * d + ch];
    const float mu = (float)(s / (double)A.n_tokens);
    A.mu[unit * d + ch] = mu;
    if (A.mean_out) A.mean_out[unit * d + ch] = mu;
  }
}

// Patterns of a chunk of tokens (index records) and per-chunk centroid sums, one sub-tile of
// kIndexSub tokens at a time, all 256 threads in every phase:
//   load     thread (token, channel octet): 16-byte loads into a padded float tile
//   pattern  thread (token, index byte): 8 comparisons with mu, one record byte
//   centroid thread (channel, slice): the slice's tokens in order, sum[slice][pattern][channel]
//            += k - mu (float64, in LDS).  Four tokens per round: their four partial sums are
//            read together and a later token of the same pattern adds to the earlier one's
//            result, so every sum still takes its tokens in order.
// The chunk's sums are the slices' sums in slice order (the tokens of a sub-tile are split
// into contiguous slices), so the result is deterministic.
template <int D, tq_dtype DT>
__global__ __launch_bounds__(256) void index_pattern_kernel(IndexArgs A) {
  constexpr int NG = D / 4, NCG = D / 8, S = 256 / D, TPS = kIndexSub / S, KS = D + 4;
  static_assert(TPS % 4 == 0, "slices take whole rounds of four tokens");
  __shared__ float mu[D];
  __shared__ __attribute__((aligned(16))) float kt[kIndexSub * KS];
  __shared__ __attribute__((aligned(4))) uint8_t pat[NG * kIndexSub];   // [group][token]
  __shared__ double acc[S * 16 * D];          // [slice][pattern][channel]
  __shared__ int32_t cnt[S * NG * 16];        // [slice][group][pattern]
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t unit = (int64_t)b * A.heads + h;
  for (int i = threadIdx.x; i < D; i += 256) mu[i] = A.mu[unit * D + i];
  for (int i = threadIdx.x; i < S * 16 * D; i += 256) acc[i] = 0.0;
  for (int i = threadIdx.x; i < S * NG * 16; i += 256) cnt[i] = 0;
  const int64_t base = (int64_t)b * A.seq_stride + (int64_t)h * A.head_stride;
  const int64_t t0 = (int64_t)chunk * A.chunk, t1 = min(A.n_tokens, t0 + A.chunk);
  const int ch = threadIdx.x % D, sl = threadIdx.x / D, g = ch / 4;
  double* as = acc + sl * 16 * D + ch;
  // the next sub-tile's keys are loaded into registers while this one is processed
  constexpr int NL = kIndexSub * NCG / 256;    // (token, octet) items per thread
  uint32_t nxt[NL][8];                         // raw, converted when stored
  auto load_tile = [&](int64_t s0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = threadIdx.x + 256 * i, tt = e / NCG, cg = e % NCG;
      load8_raw<DT>(A.k, base + min(s0 + tt, t1 - 1) * A.tok_stride + 8 * cg, nxt[i]);   // clamped
    }
  };
  if (t0 < t1) load_tile(t0);
  for (int64_t s0 = t0; s0 < t1; s0 += kIndexSub) {
    const int ns = (int)min((int64_t)kIndexSub, t1 - s0);
    __syncthreads();            // the previous sub-tile's readers are done
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = threadIdx.x + 256 * i, tt = e / NCG, cg = e % NCG;
      float v[8];
      cvt8<DT>(nxt[i], v);
      if (tt >= ns)             // rows past the sub-tile's tokens: k = mu, pattern 0 (adds 0)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = mu[8 * cg + j];
      float4* dst = reinterpret_cast<float4*>(kt + tt * KS + 8 * cg);
      dst[0] = make_float4(v[0], v[1], v[2], v[3]);
      dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
    if (s0 + kIndexSub < t1) load_tile(s0 + kIndexSub);
    __syncthreads();
    for (int e = threadIdx.x; e < kIndexSub * NCG; e += 256) {
      const int tt = e / NCG, pg = e % NCG;     // index byte pg: groups 2 pg (low nibble), 2 pg + 1
      uint32_t byte = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) byte |= (kt[tt * KS + 8 * pg + j] >= mu[8 * pg + j] ? 1u : 0u) << j;
      if (tt >= ns) byte = 0;
      pat[(2 * pg) * kIndexSub + tt] = (uint8_t)(byte & 15u);
      pat[(2 * pg + 1) * kIndexSub + tt] = (uint8_t)(byte >> 4);
      if (tt < ns) {
        int32_t* cs = cnt + (tt / TPS) * NG * 16;
        atomicAdd(&cs[(2 * pg) * 16 + (byte & 15u)], 1);
        atomicAdd(&cs[(2 * pg + 1) * 16 + (byte >> 4)], 1);
        A.index[(unit * A.capacity + A.first_slot + s0 + tt) * (D / 8) + pg] = (uint8_t)byte;
      }
    }
    __syncthreads();
    const double m = (double)mu[ch];
    for (int r = 0; r < TPS; r += 4) {
      int pp[4];
      double vv[4], old[4];
      const uint32_t p4 = *reinterpret_cast<const uint32_t*>(pat + g * kIndexSub + sl * TPS + r);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int tt = sl * TPS + r + u;
        pp[u] = (p4 >> (8 * u)) & 15u;
        vv[u] = (double)kt[tt * KS + ch] - m;   // 0 on padding rows
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) old[u] = as[pp[u] * D];
      double nw[4];
      nw[0] = old[0] + vv[0];
      nw[1] = (pp[1] == pp[0] ? nw[0] : old[1]) + vv[1];
      nw[2] = (pp[2] == pp[1] ? nw[1] : pp[2] == pp[0] ? nw[0] : old[2]) + vv[2];
      nw[3] = (pp[3] == pp[2] ? nw[2] : pp[3] == pp[1] ? nw[1] : pp[3] == pp[0] ? nw[0] : old[3]) + vv[3];
#pragma unroll
      for (int u = 0; u < 4; ++u) as[pp[u] * D] = nw[u];   // a later equal pattern's write wins
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < NG * 64; e += 256) {
    const int gg = e / 64, p = (e / 4) % 16, j = e % 4;
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < S; ++q) s += acc[(q * 16 + p) * D + 4 * gg + j];
    A.csum[((unit * A.n_chunks + chunk) * NG + gg) * 64 + p * 4 + j] = s;
  }
  for (int e = threadIdx.x; e < NG * 16; e += 256) {
    int n = 0;
#pragma unroll
    for (int q = 0; q < S; ++q) n += cnt[q * NG * 16 + e];
    A.ccnt[(unit * A.n_chunks + chunk) * NG * 16 + e] = n;
  }
}

// Patterns and per-chunk centroid sums for every other head_dim (d read at run time, a multiple
// of 8 up to 256): thread ch < d owns channel ch and takes the chunk's tokens in order - bit
// [k >= mu], the 4-bit pattern of its group and the record byte from a wave ballot (groups
// and octets never straddle a wave), then sum[pattern][ch] += k - mu in float64 (LDS), the
// group's first thread counting.  Same per-chunk sums as index_pattern_kernel.
template <tq_dtype DT>
__global__ __launch_bounds__(256) void index_pattern_generic_kernel(IndexArgs A) {
  __shared__ double acc[16 * kGenMaxD];       // [pattern][channel]
  __shared__ int32_t cnt[kGenMaxD / 4 * 16];  // [group][pattern]
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, d = A.d, ng = d / 4;
  const int ch = threadIdx.x, lane = ch & 63;
  const int64_t unit = (int64_t)b * A.heads + h;
  for (int i = threadIdx.x; i < 16 * kGenMaxD; i += 256) acc[i] = 0.0;
  for (int i = threadIdx.x; i < ng * 16; i += 256) cnt[i] = 0;
  __syncthreads();
  const bool own = ch < d;
  const float mu = own ? A.mu[unit * d + ch] : 0.0f;
  const int64_t base = (int64_t)b * A.seq_stride + (int64_t)h * A.head_stride + (own ? ch : 0);
  const int64_t t0 = (int64_t)chunk * A.chunk, t1 = min(A.n_tokens, t0 + A.chunk);
  uint8_t* idx = A.index + (unit * A.capacity + A.first_slot) * (d / 8);
  for (int64_t t = t0; t < t1; ++t) {
    const float k = load_elem(A.k, DT, base + t * A.tok_stride);
    const bool bit = own && k >= mu;
    const uint64_t bal = __ballot(bit);
    const int p = (int)((bal >> (lane & ~3)) & 15u);
    if (own) {
      acc[p * kGenMaxD + ch] += (double)k - (double)mu;
      if ((ch & 3) == 0) cnt[(ch >> 2) * 16 + p] += 1;
      if ((ch & 7) == 0) idx[t * (d / 8) + (ch >> 3)] = (uint8_t)((bal >> (lane & ~7)) & 0xFFu);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < ng * 64; e += 256) {
    const int gg = e / 64, p = (e / 4) % 16, j = e % 4;
    A.csum[((unit * A.n_chunks + chunk) * ng + gg) * 64 + p * 4 + j] = acc[p * kGenMaxD + 4 * gg + j];
  }
  for (int e = threadIdx.x; e < ng * 16; e += 256) A.ccnt[(unit * A.n_chunks + chunk) * ng * 16 + e] = cnt[e];
}

// One workgroup per (group, KV head, sequence); thread (pattern, channel) sums the chunks in
// order.
__global__ __launch_bounds__(64) void index_centroid_final_kernel(IndexArgs A) {
  const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z, ng = A.d / 4, e = threadIdx.x, p = e / 4;
  const int64_t unit = (int64_t)b * A.heads + h;
  double s = 0.0;
  int64_t n = 0;
  for (int c = 0; c < A.n_chunks; ++c) {
    s += A.csum[((unit * A.n_chunks + c) * ng + g) * 64 + e];
    n += A.ccnt[(unit * A.n_chunks + c) * ng * 16 + g * 16 + p];
  }
  A.codebook[(unit * ng + g) * 64 + e] = n > 0 ? (float)(s / (double)n) : 0.0f;
}

hipError_t launch_sign_index(const Consts& c, const IndexPlan& plan, const void* k, tq_dtype dt,
                             int batch, int64_t n_tokens, int heads, int64_t seq_stride,
                             int64_t tok_stride, int64_t head_stride, void* index, float* codebook,
                             float* mean, int64_t capacity, int64_t first_slot, void* workspace,
                             hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t units = (size_t)batch * heads;
  IndexArgs A;
  A.k = k;
  A.dt = dt;
  A.d = c.d;
  A.heads = heads;
  A.chunk = plan.chunk;
  A.n_chunks = plan.n_chunks;
  A.n_tokens = n_tokens;
  A.seq_stride = seq_stride;
  A.tok_stride = tok_stride;
  A.head_stride = head_stride;
  A.capacity = capacity;
  A.first_slot = first_slot;
  A.mean_part = reinterpret_cast<double*>(ws + plan.ws_mean);
  A.mu = reinterpret_cast<float*>(ws + plan.ws_mean + align256(units * plan.n_chunks * c.d * 8));
  A.csum = reinterpret_cast<double*>(ws + plan.ws_csum);
  A.ccnt = reinterpret_cast<int32_t*>(ws + plan.ws_ccnt);
  A.index = static_cast<uint8_t*>(index);
  A.codebook = codebook;
  A.mean_out = mean;
  dim3 grid(plan.n_chunks, heads, batch);
  if (dt == TQ_F32) hipLaunchKernelGGL(index_mean_kernel<TQ_F32>, grid, dim3(256), 0, stream, A);
  else if (dt == TQ_F16) hipLaunchKernelGGL(index_mean_kernel<TQ_F16>, grid, dim3(256), 0, stream, A);
  else hipLaunchKernelGGL(index_mean_kernel<TQ_BF16>, grid, dim3(256), 0, stream, A);
  hipLaunchKernelGGL(index_mean_final_kernel, dim3(heads, batch), dim3(128), 0, stream, A);
  if (c.d != 64 && c.d != 128) {
    if (dt == TQ_F32) hipLaunchKernelGGL(index_pattern_generic_kernel<TQ_F32>, grid, dim3(256), 0, stream, A);
    else if (dt == TQ_F16) hipLaunchKernelGGL(index_pattern_generic_kernel<TQ_F16>, grid, dim3(256), 0, stream, A);
    else hipLaunchKernelGGL(index_pattern_generic_kernel<TQ_BF16>, grid, dim3(256), 0, stream, A);
  } else if (c.d == 128 && dt == TQ_F32) hipLaunchKernelGGL((index_pattern_kernel<128, TQ_F32>), grid, dim3(256), 0, stream, A);
  else if (c.d == 128 && dt == TQ_F16) hipLaunchKernelGGL((index_pattern_kernel<128, TQ_F16>), grid, dim3(256), 0, stream, A);
  else if (c.d == 128) hipLaunchKernelGGL((index_pattern_kernel<128, TQ_BF16>), grid, dim3(256), 0, stream, A);
  else if (dt == TQ_F32) hipLaunchKernelGGL((index_pattern_kernel<64, TQ_F32>), grid, dim3(256), 0, stream, A);
  else if (dt == TQ_F16) hipLaunchKernelGGL((index_pattern_kernel<64, TQ_F16>), grid, dim3(256), 0, stream, A);
  else hipLaunchKernelGGL((index_pattern_kernel<64, TQ_BF16>), grid, dim3(256), 0, stream, A);
  hipLaunchKernelGGL(index_centroid_final_kernel, dim3(c.d / 4, heads, batch), dim3(64), 0, stream, A);
  return hipGetLastError();
}

// =========================================================================================
// Top-k selection from the sign index (Self-Indexing page, "Methodologie" 3, LUT-GEMV).
// LUT[h][g][p] = ((q0 c0 + q1 c1) + q2 c2) + q3 c3 in float64 (no fused multiply-add, so the
// rounding is fixed), s = largest integer with G (d/4) max|LUT| 2^s <= 2^30, entries
// rint(LUT 2^s) (half to even) summed over the group's heads: integer scores, exact and
// independent of summation order.  Ranking: score descending, then token index ascending.
// =========================================================================================
constexpr int kSelBinsTotal = 4096;       // histogram bins per unit (top 12 bits of the order key)

SelectPlan plan_select(const Consts& c, int batch, int heads, int64_t capacity) {
  SelectPlan p;
  const size_t units = (size_t)std::max(batch, 1) * heads;
  const size_t cap = (size_t)std::max<int64_t>(capacity, 1);
  p.n_chunks = (int)((cap + 4095) / 4096);
  p.ws_lut = 0;                                                       // i32 [units][d/4][16]
  p.ws_scores = p.ws_lut + align256(units * (c.d / 4) * 16 * 4);      // i32 [units][capacity]
  p.ws_hist = p.ws_scores + align256(units * cap * 4);                // i32 [units][4096]
  p.ws_cand = p.ws_hist + align256(units * kSelBinsTotal * 4);        // u32x2 [units][capacity]:
                                                                      // chunk c's candidates at 4096 c
  p.ws_chunk_cand = p.ws_cand + align256(units * cap * 8);            // i32 [units][n_chunks]
  p.ws_chunk_above = p.ws_chunk_cand + align256(units * p.n_chunks * 4);
  p.ws_chunk_off = p.ws_chunk_above + align256(units * p.n_chunks * 4);
  p.ws_params = p.ws_chunk_off + align256(units * p.n_chunks * 4);    // 24 B [units]
  p.ws_total = p.ws_params + align256(units * 32);
  return p;
}

__device__ __forceinline__ double lut_entry(double q0, double q1, double q2, double q3, const float* cen) {
#pragma clang fp contract(off)
  double t = q0 * (double)cen[0];
  t = t + q1 * (double)cen[1];
  t = t + q2 * (double)cen[2];
  t = t + q3 * (double)cen[3];
  return t;
}

__device__ __forceinline__ void select_lut_block(const void* q, tq_dtype q_dt, const float* codebook, int d, int G,
                                                 int q_heads, int heads, int32_t* lut_out, int32_t* hist_all,
                                                 int h, int b) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int ng = d / 4;
  const int64_t unit = (int64_t)b * heads + h;
  double* lut = reinterpret_cast<double*>(smem);           // [G][ng][16]
  int32_t* comb = reinterpret_cast<int32_t*>(lut + G * ng * 16);  // [ng][16]
  __shared__ double mx[16];                                 // one per wave, up to 1,024 threads
  const float* cb = codebook + unit * ng * 64;
  for (int e = threadIdx.x; e < kSelBinsTotal; e += blockDim.x) hist_all[unit * kSelBinsTotal + e] = 0;
  double m = 0.0;
  for (int e = threadIdx.x; e < G * ng * 16; e += blockDim.x) {
    const int j = e / (ng * 16), g = (e / 16) % ng, p = e % 16;
    const int64_t qrow = ((int64_t)b * q_heads + (int64_t)h * G + j) * d + 4 * g;
    const double v = lut_entry((double)load_elem(q, q_dt, qrow), (double)load_elem(q, q_dt, qrow + 1),
                               (double)load_elem(q, q_dt, qrow + 2), (double)load_elem(q, q_dt, qrow + 3),
                               cb + g * 64 + p * 4);
    lut[e] = v;
    m = fmax(m, fabs(v));
  }
  // block max: wave shuffles, then one LDS word per wave
#pragma unroll
  for (int msk = 32; msk > 0; msk >>= 1) m = fmax(m, __shfl_xor(m, msk));
  if ((threadIdx.x & 63) == 0) mx[threadIdx.x >> 6] = m;
  __syncthreads();
  double mall = mx[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) mall = fmax(mall, mx[w]);
  const double a = (double)(G * ng) * mall;
  int sexp = 0;
  if (a != 0.0) {
    int e;
    const double f = frexp(a, &e);
    sexp = 30 - e + (f == 0.5 ? 1 : 0);
  }
  for (int e = threadIdx.x; e < ng * 16; e += blockDim.x) {
    int64_t s = 0;
    for (int j = 0; j < G; ++j) s += (int64_t)rint(ldexp(lut[j * ng * 16 + e], sexp));
    comb[e] = (int32_t)s;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < ng * 16; e += blockDim.x) lut_out[unit * ng * 16 + e] = comb[e];
}

__global__ __launch_bounds__(256) void select_lut_kernel(const void* q, tq_dtype q_dt, const float* codebook,
                                                         int d, int G, int q_heads, int heads,
                                                         int32_t* lut_out, int32_t* hist_all) {
  select_lut_block(q, q_dt, codebook, d, G, q_heads, heads, lut_out, hist_all, blockIdx.x, blockIdx.y);
}

// The selection tables and the attention's query prep in one launch (sparse attention, whose
// two first steps are independent one-block-per-unit / per-query jobs): blocks below
// batch * heads build a unit's tables, the others prepare query row blockIdx.x - batch * heads.
__global__ __launch_bounds__(kQueryPrepThreads) void select_lut_prep_kernel(const void* q, tq_dtype q_dt, const float* codebook,
                                                              int d, int G, int q_heads, int heads, int units,
                                                              int32_t* lut_out, int32_t* hist_all, QueryPrep P) {
  if ((int)blockIdx.x < units)
    select_lut_block(q, q_dt, codebook, d, G, q_heads, heads, lut_out, hist_all, blockIdx.x % heads,
                     blockIdx.x / heads);
  else
    query_prep_block(P.pi, P.s, d, P.m, q, q_dt, P.qx, P.qs, (int64_t)blockIdx.x - units);
}

// Selection runs in five launches (lut and exact: one workgroup per unit; score, filter and
// write: one workgroup per 4096-token chunk of every unit):
//   lut    (unit)          per-query byte tables; clears the unit's histogram
//   score  (chunk, unit)   integer score of each token, stored; 4096-bin histogram of the top
//                          12 bits of the order key, merged into the unit's histogram
//   filter (chunk, unit)   finds the bin B holding the k-th largest score; counts the chunk's
//                          tokens above B and writes the tokens in B to its own candidate
//                          region (slots 4096 c onwards; LDS counter, no global atomics)
//   exact  (unit)          radix passes over the candidates on the 64-bit key
//                          (order key << 32 | ~index), unique per token, so that exactly k tokens
//                          satisfy (key & M) >= P; per-chunk counts -> output offsets
//   write  (chunk, unit)   ordered compaction of the chunk's selected tokens at its offset
// The composite key ranks score descending then index ascending, the oracle's order.
constexpr int kSelChunk = 4096;           // tokens per workgroup in score / filter / write
constexpr int kSelBins = kSelBinsTotal;
constexpr int kSelDigitShift = 20;
constexpr int kSelExactThreads = 1024;

__device__ __forceinline__ uint32_t order_key(int32_t s) { return (uint32_t)s ^ 0x80000000u; }

__device__ __forceinline__ uint64_t select_key(uint32_t u, int32_t t) {
  return ((uint64_t)u << 32) | (uint64_t)(~(uint32_t)t);
}

// Exclusive prefix sum over the block of one value per thread; *total gets the block sum.
template <int NT>
__device__ __forceinline__ int block_exclusive_sum(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    off += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  *total = tot;
  return off + incl - v;
}

// 512 threads of 8 tokens each (two batches of 4 records in flight, ~48 VGPRs): all 4,096-token
// chunks of the sparse workload are resident at once (8 waves per SIMD), hiding the record loads
// and table reads better than 256 threads of 16 tokens (17.6 against 19.4 us at 131,072 tokens).
constexpr int kScoreThreads = 512;

template <int NB>
__global__ __launch_bounds__(kScoreThreads, 8) void select_score_kernel(const uint8_t* index, const int32_t* lut_all,
                                                           const int32_t* seq_lens, int heads, int64_t capacity,
                                                           int32_t* scores, int32_t* hist_all) {
  // one 16-entry table per 4-channel group: a lookup instruction reads one table, whose 16
  // words sit in 16 distinct banks, so lookups never conflict (equal patterns broadcast)
  constexpr int NG = 2 * NB;
  __shared__ int32_t lut[NG * 16];
  __shared__ int32_t hist[kSelBins];
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t unit = (int64_t)b * heads + h;
  const int64_t n = min((int64_t)seq_lens[b], capacity);
  const int64_t t0 = (int64_t)blockIdx.x * kSelChunk;
  if (t0 >= n) return;
  for (int e = threadIdx.x; e < NG * 16; e += kScoreThreads) lut[e] = lut_all[unit * NG * 16 + e];
  for (int e = threadIdx.x; e < kSelBins; e += kScoreThreads) hist[e] = 0;
  __syncthreads();
  const uint8_t* base = index + (unit * capacity + t0) * NB;
  int32_t* sc = scores + unit * capacity + t0;
  const int m = (int)min((int64_t)kSelChunk, n - t0);
  using Rec = typename std::conditional<NB == 16, uint4, uint2>::type;
  constexpr int kBatch = 4;
  for (int i0 = 0; i0 < kSelChunk / kScoreThreads; i0 += kBatch) {
    Rec r[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int t = (i0 + j) * kScoreThreads + threadIdx.x;
      r[j] = *reinterpret_cast<const Rec*>(base + (size_t)min(t, m - 1) * NB);   // clamped, unbranched
    }
    // every token of the batch is scored (a clamped one twice) and only the store and the
    // histogram count are predicated: a branch around the whole body lets the compiler sink
    // each record load into it, which serialises the loads' latency token by token
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int t = (i0 + j) * kScoreThreads + threadIdx.x;
      uint32_t w[NB / 4];
      if constexpr (NB == 16) {
        w[0] = r[j].x; w[1] = r[j].y; w[2] = r[j].z; w[3] = r[j].w;
      } else {
        w[0] = r[j].x; w[1] = r[j].y;
      }
      // index byte k holds groups 2 k (low nibble) and 2 k + 1; nibbles pre-scaled to byte
      // offsets within a table, so each lookup address is one byte extract
      const uint8_t* lb = reinterpret_cast<const uint8_t*>(lut);
      int32_t s = 0;
#pragma unroll
      for (int i = 0; i < NB / 4; ++i) {
        uint32_t lo = (w[i] << 2) & 0x3C3C3C3Cu, hi = (w[i] >> 2) & 0x3C3C3C3Cu;
        asm volatile("" : "+v"(lo));
        asm volatile("" : "+v"(hi));
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int g = 2 * (4 * i + kb);
          s += *reinterpret_cast<const int32_t*>(lb + 64 * g + ((lo >> (8 * kb)) & 0xFFu));
          s += *reinterpret_cast<const int32_t*>(lb + 64 * (g + 1) + ((hi >> (8 * kb)) & 0xFFu));
        }
      }
      if (t < m) {
        sc[t] = s;
        atomicAdd(&hist[order_key(s) >> kSelDigitShift], 1);
      }
    }
  }
  __syncthreads();
  int32_t* gh = hist_all + unit * kSelBins;
  for (int e = threadIdx.x; e < kSelBins; e += kScoreThreads) {
    const int v = hist[e];
    if (v) atomicAdd(&gh[e], v);
  }
}

// Scores for every other head_dim: index records of d / 8 bytes read byte by byte, one
// 16-entry table per 4-channel group (d / 4 groups), 16 tokens per thread; the same histogram.
__global__ __launch_bounds__(256) void select_score_generic_kernel(const uint8_t* index, const int32_t* lut_all,
                                                                   const int32_t* seq_lens, int heads, int d,
                                                                   int64_t capacity, int32_t* scores,
                                                                   int32_t* hist_all) {
  __shared__ int32_t lut[kGenMaxD / 4 * 16];
  __shared__ int32_t hist[kSelBins];
  const int h = blockIdx.y, b = blockIdx.z, ng = d / 4, nb = d / 8;
  const int64_t unit = (int64_t)b * heads + h;
  const int64_t n = min((int64_t)seq_lens[b], capacity);
  const int64_t t0 = (int64_t)blockIdx.x * kSelChunk;
  if (t0 >= n) return;
  for (int e = threadIdx.x; e < ng * 16; e += 256) lut[e] = lut_all[unit * ng * 16 + e];
  for (int e = threadIdx.x; e < kSelBins; e += 256) hist[e] = 0;
  __syncthreads();
  const uint8_t* base = index + (unit * capacity + t0) * nb;
  int32_t* sc = scores + unit * capacity + t0;
  const int m = (int)min((int64_t)kSelChunk, n - t0);
  for (int t = threadIdx.x; t < m; t += 256) {
    const uint8_t* r = base + (int64_t)t * nb;
    int32_t s = 0;
    for (int k = 0; k < nb; ++k) {
      const uint32_t byte = r[k];
      s += lut[(2 * k) * 16 + (byte & 15u)] + lut[(2 * k + 1) * 16 + (byte >> 4)];
    }
    sc[t] = s;
    atomicAdd(&hist[order_key(s) >> kSelDigitShift], 1);
  }
  __syncthreads();
  int32_t* gh = hist_all + unit * kSelBins;
  for (int e = threadIdx.x; e < kSelBins; e += 256) {
    const int v = hist[e];
    if (v) atomicAdd(&gh[e], v);
  }
}

struct SelectParams {
  uint32_t bin, above;                    // bin of the k-th score; tokens in higher bins
  uint64_t prefix, mask;                  // selected iff (select_key & mask) >= prefix
};

__global__ __launch_bounds__(256) void select_filter_kernel(const int32_t* scores, const int32_t* hist_all,
                                                            const int32_t* seq_lens, int heads, int64_t capacity,
                                                            int k, int n_chunks, uint2* cand_all,
                                                            int32_t* chunk_cand, int32_t* chunk_above,
                                                            SelectParams* params) {
  __shared__ int wsum[4];
  __shared__ uint32_t s_bin, s_above;
  __shared__ int s_ncand;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t unit = (int64_t)b * heads + h;
  const int64_t n = min((int64_t)seq_lens[b], capacity);
  const int64_t kk = min((int64_t)k, n);
  const int64_t t0 = (int64_t)blockIdx.x * kSelChunk;
  if (kk == 0 || kk == n || t0 >= n) return;
  if (threadIdx.x == 0) s_ncand = 0;
  // bin holding the kk-th largest key: thread i owns bins [16 i, 16 i + 16), higher threads
  // hold higher bins; an exclusive sum over the reversed thread order counts what lies above.
  const int32_t* gh = hist_all + unit * kSelBins;
  const int32_t* sc = scores + unit * capacity + t0;
  const int m = (int)min((int64_t)kSelChunk, n - t0);
  // the chunk's scores are loaded first, so their latency overlaps the bin search
  uint32_t u[kSelChunk / 256];
#pragma unroll
  for (int i = 0; i < kSelChunk / 256; ++i) {
    const int t = i * 256 + threadIdx.x;
    const uint32_t v = order_key(sc[min(t, m - 1)]);      // clamped: no branch around the load
    u[i] = t < m ? v : 0u;
  }
  int own = 0;
  int hv[16];
#pragma unroll
  for (int j = 0; j < 16; j += 4) {
    const int4 v = *reinterpret_cast<const int4*>(gh + 16 * threadIdx.x + j);
    hv[j] = v.x; hv[j + 1] = v.y; hv[j + 2] = v.z; hv[j + 3] = v.w;
    own += v.x + v.y + v.z + v.w;
  }
  // count above thread i's bins = exclusive sum over slots in reversed thread order
  // (slot j holds thread 255 - j)
  __shared__ int owns[256];
  int tot;
  const int rev = 255 - (int)threadIdx.x;
  owns[rev] = own;
  __syncthreads();
  const int ex = block_exclusive_sum<256>(owns[threadIdx.x], wsum, &tot);
  __syncthreads();
  owns[threadIdx.x] = ex;         // count above the bins of thread 255 - threadIdx.x
  __syncthreads();
  {
    const int above = owns[rev];
    if (above < kk && above + own >= kk) {
      int cum = above;
      for (int j = 15; j >= 0; --j) {
        if (cum + hv[j] >= kk) {
          s_bin = 16u * threadIdx.x + (uint32_t)j;
          s_above = (uint32_t)cum;
          break;
        }
        cum += hv[j];
      }
    }
  }
  __syncthreads();
  const uint32_t bin = s_bin;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    params[unit].bin = bin;
    params[unit].above = s_above;
  }
  uint2* cand = cand_all + unit * capacity + t0;   // this chunk's candidate region
  const int lane = threadIdx.x & 63;
  int cnt_above = 0;
#pragma unroll
  for (int i = 0; i < kSelChunk / 256; ++i) {
    const int t = i * 256 + threadIdx.x;
    const uint32_t dig = u[i] >> kSelDigitShift;
    const bool in = t < m;
    cnt_above += (in && dig > bin) ? 1 : 0;
    const bool eq = in && dig == bin;
    const uint64_t bal = __ballot(eq);
    if (bal) {
      const int leader = __ffsll((long long)bal) - 1;
      int basepos = 0;
      if (lane == leader) basepos = atomicAdd(&s_ncand, __popcll(bal));   // LDS counter
      basepos = __shfl(basepos, leader);
      if (eq) cand[basepos + __popcll(bal & ((1ull << lane) - 1ull))] = make_uint2(u[i], (uint32_t)(t0 + t));
    }
  }
  (void)block_exclusive_sum<256>(cnt_above, wsum, &tot);   // (its barriers also settle s_ncand)
  if (threadIdx.x == 0) {
    chunk_above[unit * n_chunks + blockIdx.x] = tot;
    chunk_cand[unit * n_chunks + blockIdx.x] = s_ncand;
  }
}

__global__ __launch_bounds__(kSelExactThreads) void select_exact_kernel(
    const int32_t* seq_lens, int heads, int64_t capacity, int k, int n_chunks, const uint2* cand_all,
    const int32_t* chunk_cand, const int32_t* chunk_above, int32_t* chunk_off, SelectParams* params,
    int32_t* out_idx, int32_t* out_count, int32_t* out_scores) {
  extern __shared__ int32_t chunk_cnt[];          // [n_chunks] selected counts, then [n_chunks]
                                                  // exclusive prefix of candidate counts
  __shared__ int hist[256];
  __shared__ int wsum[kSelExactThreads / 64];
  __shared__ uint32_t s_digit, s_rem, s_cnt;
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t unit = (int64_t)b * heads + h;
  const int64_t n = min((int64_t)seq_lens[b], capacity);
  const int64_t kk = min((int64_t)k, n);
  if (out_count && threadIdx.x == 0) out_count[unit] = (int32_t)kk;
  if (out_idx)
    for (int64_t i = kk + threadIdx.x; i < k; i += blockDim.x) {
      out_idx[unit * k + i] = -1;
      if (out_scores) out_scores[unit * k + i] = 0;
    }
  if (kk == 0) return;
  const int nch = (int)((n + kSelChunk - 1) / kSelChunk);
  int32_t* off = chunk_off + unit * n_chunks;
  if (kk == n) {
    for (int c = threadIdx.x; c < nch; c += blockDim.x) off[c] = c * kSelChunk;
    if (threadIdx.x == 0) {
      params[unit].prefix = 0;
      params[unit].mask = 0;
    }
    return;
  }
  const uint2* cand = cand_all + unit * capacity;
  // candidate i lives in the region of chunk c = last chunk with cpre[c] <= i
  int32_t* cpre = chunk_cnt + n_chunks;
  int nc = 0;
  for (int c0 = 0; c0 < nch; c0 += blockDim.x) {
    const int c = c0 + threadIdx.x;
    const int v = c < nch ? chunk_cand[unit * n_chunks + c] : 0;
    int tot;
    const int ex = block_exclusive_sum<kSelExactThreads>(v, wsum, &tot);
    if (c < nch) cpre[c] = nc + ex;
    nc += tot;
  }
  __syncthreads();
  auto cand_at = [&](int i) {
    int lo = 0, hi = nch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cpre[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return cand[(int64_t)lo * kSelChunk + (i - cpre[lo])];
  };
  const SelectParams p0 = params[unit];
  uint64_t prefix = (uint64_t)p0.bin << (32 + kSelDigitShift);
  uint64_t mask = (uint64_t)(kSelBins - 1) << (32 + kSelDigitShift);
  uint32_t rem = (uint32_t)(kk - p0.above);
  uint32_t cnt = (uint32_t)nc;                 // candidates matching the prefix
  // digit fields below the 12 histogrammed bits: order-key bits 19..12, 11..4, 3..0 (key bits
  // 51..32), then the inverted index in four bytes (key bits 31..0)
  for (int pass = 0; pass < 7 && cnt != rem; ++pass) {
    const int sh = pass < 2 ? 44 - 8 * pass : (pass == 2 ? 32 : 24 - 8 * (pass - 3));
    const uint32_t dm = pass == 2 ? 15u : 255u;
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < nc; i += blockDim.x) {
      const uint2 cu = cand_at(i);
      const uint64_t key = select_key(cu.x, (int32_t)cu.y);
      if ((key & mask) == prefix) atomicAdd(&hist[(uint32_t)(key >> sh) & dm], 1);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l owns digits [4 l, 4 l + 4); inclusive suffix sums over the lanes above
      const int l = threadIdx.x;
      const int own = hist[4 * l] + hist[4 * l + 1] + hist[4 * l + 2] + hist[4 * l + 3];
      int suf = own;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_down(suf, o);
        if (l + o < 64) suf += v;
      }
      const int above = suf - own;
      if (above < (int)rem && suf >= (int)rem) {
        int cum = above;
        for (int j = 3; j >= 0; --j) {
          const int hvv = hist[4 * l + j];
          if (cum + hvv >= (int)rem) {
            s_digit = (uint32_t)(4 * l + j);
            s_rem = rem - (uint32_t)cum;
            s_cnt = (uint32_t)hvv;
            break;
          }
          cum += hvv;
        }
      }
    }
    __syncthreads();
    prefix |= (uint64_t)s_digit << sh;
    mask |= (uint64_t)dm << sh;
    rem = s_rem;
    cnt = s_cnt;
    __syncthreads();
  }
  // per-chunk selected counts, then exclusive offsets
  for (int c = threadIdx.x; c < nch; c += blockDim.x) chunk_cnt[c] = chunk_above[unit * n_chunks + c];
  __syncthreads();
  for (int i = threadIdx.x; i < nc; i += blockDim.x) {
    const uint2 cu = cand_at(i);
    if ((select_key(cu.x, (int32_t)cu.y) & mask) >= prefix) atomicAdd(&chunk_cnt[cu.y / kSelChunk], 1);
  }
  __syncthreads();
  int carry = 0;
  for (int c0 = 0; c0 < nch; c0 += blockDim.x) {
    const int c = c0 + threadIdx.x;
    const int v = c < nch ? chunk_cnt[c] : 0;
    int tot;
    const int ex = block_exclusive_sum<kSelExactThreads>(v, wsum, &tot);
    if (c < nch) off[c] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) {
    params[unit].prefix = prefix;
    params[unit].mask = mask;
  }
}

__global__ __launch_bounds__(256) void select_write_kernel(const int32_t* scores, const int32_t* seq_lens, int heads,
                                                           int64_t capacity, int k, int n_chunks,
                                                           const int32_t* chunk_off, const SelectParams* params,
                                                           int32_t* out_idx, int32_t* out_scores) {
  __shared__ int wsum[4];
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t unit = (int64_t)b * heads + h;
  const int64_t n = min((int64_t)seq_lens[b], capacity);
  const int64_t kk = min((int64_t)k, n);
  const int64_t t0 = (int64_t)blockIdx.x * kSelChunk;
  if (kk == 0 || t0 >= n) return;
  const uint64_t prefix = params[unit].prefix, mask = params[unit].mask;
  const int32_t* sc = scores + unit * capacity + t0;
  const int m = (int)min((int64_t)kSelChunk, n - t0);
  constexpr int kPer = kSelChunk / 256;
  const int tb = (int)threadIdx.x * kPer;        // this thread's tokens [tb, tb + 16) in index order
  int32_t s[kPer];
  if (tb + kPer <= m) {
#pragma unroll
    for (int j = 0; j < kPer; j += 4) {
      const int4 v = *reinterpret_cast<const int4*>(sc + tb + j);
      s[j] = v.x; s[j + 1] = v.y; s[j + 2] = v.z; s[j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) s[j] = tb + j < m ? sc[tb + j] : 0;
  }
  uint32_t sel = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int t = tb + j;
    const bool take = t < m && (select_key(order_key(s[j]), (int32_t)(t0 + t)) & mask) >= prefix;
    sel |= (take ? 1u : 0u) << j;
  }
  int tot;
  int pos = chunk_off[unit * n_chunks + blockIdx.x] + block_exclusive_sum<256>(__popc(sel), wsum, &tot);
  int32_t* oi = out_idx + unit * k;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if ((sel & (1u << j)) && pos < kk) {
      oi[pos] = (int32_t)(t0 + tb + j);
      if (out_scores) out_scores[unit * k + pos] = s[j];
      ++pos;
    }
  }
}

hipError_t launch_select(const Consts& c, const SelectPlan& plan, const void* q, tq_dtype q_dt, int batch,
                         int q_heads, int kv_heads, const void* index, const float* codebook,
                         int64_t capacity, const int32_t* seq_lens, int k, int32_t* out_idx,
                         int32_t* out_count, int32_t* out_scores, void* workspace, hipStream_t stream,
                         const ProfileEvents& ev, const QueryPrep* prep, bool skip_exact) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* lut = reinterpret_cast<int32_t*>(ws + plan.ws_lut);
  int32_t* scores = reinterpret_cast<int32_t*>(ws + plan.ws_scores);
  int32_t* hist = reinterpret_cast<int32_t*>(ws + plan.ws_hist);
  uint2* cand = reinterpret_cast<uint2*>(ws + plan.ws_cand);
  int32_t* chunk_cand = reinterpret_cast<int32_t*>(ws + plan.ws_chunk_cand);
  int32_t* chunk_above = reinterpret_cast<int32_t*>(ws + plan.ws_chunk_above);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(ws + plan.ws_chunk_off);
  SelectParams* params = reinterpret_cast<SelectParams*>(ws + plan.ws_params);
  const int G = q_heads / kv_heads, ng = c.d / 4;
  const int n_chunks = plan.n_chunks;
  if (capacity > 0) {
    const size_t lds = (size_t)G * ng * 16 * 8 + (size_t)ng * 16 * 4;
    if (prep)
      hipLaunchKernelGGL(select_lut_prep_kernel, dim3((unsigned)(batch * kv_heads + prep->rows)), dim3(kQueryPrepThreads), lds,
                         stream, q, q_dt, codebook, c.d, G, q_heads, kv_heads, batch * kv_heads, lut, hist, *prep);
    else
      hipLaunchKernelGGL(select_lut_kernel, dim3(kv_heads, batch), dim3(256), lds, stream, q, q_dt, codebook,
                         c.d, G, q_heads, kv_heads, lut, hist);
    const dim3 grid((unsigned)n_chunks, kv_heads, batch);
    ev.before(stream);
    if (c.d != 64 && c.d != 128)
      hipLaunchKernelGGL(select_score_generic_kernel, grid, dim3(256), 0, stream, static_cast<const uint8_t*>(index),
                         lut, seq_lens, kv_heads, c.d, capacity, scores, hist);
    else if (c.d == 128)
      hipLaunchKernelGGL(select_score_kernel<16>, grid, dim3(kScoreThreads), 0, stream, static_cast<const uint8_t*>(index),
                         lut, seq_lens, kv_heads, capacity, scores, hist);
    else
      hipLaunchKernelGGL(select_score_kernel<8>, grid, dim3(kScoreThreads), 0, stream, static_cast<const uint8_t*>(index),
                         lut, seq_lens, kv_heads, capacity, scores, hist);
    ev.after(stream);
    hipLaunchKernelGGL(select_filter_kernel, grid, dim3(256), 0, stream, scores, hist, seq_lens, kv_heads, capacity,
                       k, n_chunks, cand, chunk_cand, chunk_above, params);
  }
  if (skip_exact) return hipGetLastError();     // sparse attention forms the threshold itself
  const size_t exact_lds = (size_t)std::max(n_chunks, 1) * 8;
  allow_lds(select_exact_kernel, exact_lds);
  hipLaunchKernelGGL(select_exact_kernel, dim3(kv_heads, batch), dim3(kSelExactThreads), exact_lds, stream, seq_lens, kv_heads, capacity, k, n_chunks, cand,
                     chunk_cand, chunk_above, chunk_off, params, out_idx, out_count, out_scores);
  if (capacity > 0 && k > 0 && out_idx)
    hipLaunchKernelGGL(select_write_kernel, dim3((unsigned)n_chunks, kv_heads, batch), dim3(256), 0, stream, scores,
                       seq_lens, kv_heads, capacity, k, n_chunks, chunk_off, params, out_idx, out_scores);
  return hipGetLastError();
}

// =========================================================================================
// Sparse attention in one pass over the selection (Self-Indexing page, "Methodologie" 3-5):
// after the selection's lut / score / filter / exact launches, every 4,096-token chunk of a
// (sequence, KV head) re-derives its selected tokens from the stored scores and the unit's
// predicate (the write launch's rule, including its cap at k), and attends to them directly:
// their codes are unpacked into LDS 64 tokens at a time, the G heads' estimates formed from
// q_x / q_s and the level tables, and an online softmax with the value sums kept per (head,
// coordinate); the chunk's partial (m, l, o_x) then goes through the decode merge, with the
// exact segment (e.g. sink tokens) in the same softmax.  No index list is materialised.
// =========================================================================================
struct SparseArgs {
  DecodeArgs a;             // records, layout, qx / qs, levels, scale, part, n_chunks (= select chunks)
  const int32_t* scores;    // [units][capacity] selection scores
  const SelectParams* params;
  const int32_t* chunk_off;
  // the threshold is formed by the attention (no exact launch): the filter launch's candidates
  // and per-chunk counts
  const uint2* cand_all;
  const int32_t* chunk_cand;
  const int32_t* chunk_above;
  int k;
};

// The unit's selection predicate ((key & mask) >= prefix) and the output offset of chunk c,
// formed by the attention workgroup itself from the filter launch's candidates - the exact
// launch's computation, repeated by every chunk of the unit instead of a launch of its own:
// radix passes over the candidates (the tokens in the bin of the k-th score) on the 64-bit key
// until exactly the tokens still needed match, then the tokens above the bin and the chosen
// candidates in the chunks before c.  Called by all kSmallThreads threads; the results are
// valid in every thread on return.  Needs n_chunks ints of dynamic LDS (the exclusive prefix of
// the chunks' candidate counts).
constexpr int kCandCache = 512;   // threshold candidates kept in LDS

__device__ void sparse_unit_threshold(const SparseArgs& S, int64_t unit, int c, int64_t n, int64_t kk,
                                      uint64_t* prefix_out, uint64_t* mask_out, int* base_out) {
  constexpr int NT = kSmallThreads;
  extern __shared__ int cpre[];
  __shared__ int hist[256];
  __shared__ int wsum2[NT / 64];
  __shared__ uint32_t s_digit, s_rem, s_cnt;
  const int tid = threadIdx.x;
  if (kk == 0 || kk == n) {           // nothing, or every token, is selected
    *prefix_out = 0;
    *mask_out = 0;
    *base_out = c * kSelChunk;
    return;
  }
  const int nch = (int)((n + kSelChunk - 1) / kSelChunk);
  const int32_t* ccand = S.chunk_cand + unit * S.a.n_chunks;
  const int32_t* cabove = S.chunk_above + unit * S.a.n_chunks;
  int nc = 0;
  for (int c0 = 0; c0 < nch; c0 += NT) {
    const int cc = c0 + tid;
    const int v = cc < nch ? ccand[cc] : 0;
    int tot;
    const int ex = block_exclusive_sum<NT>(v, wsum2, &tot);
    if (cc < nch) cpre[cc] = nc + ex;
    nc += tot;
  }
  __syncthreads();
  const uint2* cand = S.cand_all + unit * S.a.capacity;
  auto cand_global = [&](int i) {
    int lo = 0, hi = nch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cpre[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return cand[(int64_t)lo * kSelChunk + (i - cpre[lo])];
  };
  // the unit's candidates (the tokens in the k-th score's bin, ~100 at 131,072 tokens) are read
  // from memory once into LDS when they fit; the radix passes and the final count then read LDS
  __shared__ uint2 ccache[kCandCache];
  const bool cached = nc <= kCandCache;
  if (cached) {
    for (int i = tid; i < nc; i += NT) ccache[i] = cand_global(i);
    __syncthreads();
  }
  auto cand_at = [&](int i) { return cached ? ccache[i] : cand_global(i); };
  const SelectParams p0 = S.params[unit];
  uint64_t prefix = (uint64_t)p0.bin << (32 + kSelDigitShift);
  uint64_t mask = (uint64_t)(kSelBins - 1) << (32 + kSelDigitShift);
  uint32_t rem = (uint32_t)(kk - p0.above);
  uint32_t cnt = (uint32_t)nc;
  for (int pass = 0; pass < 7 && cnt != rem; ++pass) {
    const int sh = pass < 2 ? 44 - 8 * pass : (pass == 2 ? 32 : 24 - 8 * (pass - 3));
    const uint32_t dm = pass == 2 ? 15u : 255u;
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < nc; i += NT) {
      const uint2 cu = cand_at(i);
      const uint64_t key = select_key(cu.x, (int32_t)cu.y);
      if ((key & mask) == prefix) atomicAdd(&hist[(uint32_t)(key >> sh) & dm], 1);
    }
    __syncthreads();
    if (tid < 64) {
      const int l = tid;
      const int own = hist[4 * l] + hist[4 * l + 1] + hist[4 * l + 2] + hist[4 * l + 3];
      int suf = own;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_down(suf, o);
        if (l + o < 64) suf += v;
      }
      const int above = suf - own;
      if (above < (int)rem && suf >= (int)rem) {
        int cum = above;
        for (int j = 3; j >= 0; --j) {
          const int hvv = hist[4 * l + j];
          if (cum + hvv >= (int)rem) {
            s_digit = (uint32_t)(4 * l + j);
            s_rem = rem - (uint32_t)cum;
            s_cnt = (uint32_t)hvv;
            break;
          }
          cum += hvv;
        }
      }
    }
    __syncthreads();
    prefix |= (uint64_t)s_digit << sh;
    mask |= (uint64_t)dm << sh;
    rem = s_rem;
    cnt = s_cnt;
    __syncthreads();
  }
  int mine = 0;
  for (int i = tid; i < nc; i += NT) {
    const uint2 cu = cand_at(i);
    if ((int)(cu.y / kSelChunk) < c && (select_key(cu.x, (int32_t)cu.y) & mask) >= prefix) ++mine;
  }
  for (int cc = tid; cc < c; cc += NT) mine += cabove[cc];
  int tot;
  (void)block_exclusive_sum<NT>(mine, wsum2, &tot);
  *prefix_out = prefix;
  *mask_out = mask;
  *base_out = tot;
}

// The selected tokens of chunk c of a unit, in index order and capped at k overall (the write
// launch's rule): offsets within the chunk into list[], their count into *s_nsel (written by
// thread 0; read after the caller's next barrier).  Called by all kSmallThreads threads.
__device__ __forceinline__ void sparse_chunk_list(const SparseArgs& S, int64_t unit, int c, int64_t n,
                                                  int64_t kk, uint16_t* list, int* wsum, int* s_nsel) {
  constexpr int kPer = kSelChunk / kSmallThreads;
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)c * kSelChunk;
  const int tb = tid * kPer;
  // the chunk's scores are loaded before the threshold is formed, so that their latency overlaps
  // the threshold's own reads
  const int mm = (int)max<int64_t>(0, min((int64_t)kSelChunk, n - t0));
  int32_t s[kPer];
  if (kk > 0 && t0 < n) {
    const int32_t* sc = S.scores + unit * S.a.capacity + t0;
    if (tb + kPer <= mm) {
#pragma unroll
      for (int j = 0; j < kPer; j += 4) {
        const int4 v = *reinterpret_cast<const int4*>(sc + tb + j);
        s[j] = v.x; s[j + 1] = v.y; s[j + 2] = v.z; s[j + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kPer; ++j) s[j] = tb + j < mm ? sc[tb + j] : 0;
    }
  }
  uint64_t prefix = 0, mask = 0;
  int base = 0;
  sparse_unit_threshold(S, unit, c, n, kk, &prefix, &mask, &base);
  uint32_t sel = 0;
  if (kk > 0 && t0 < n) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int t = tb + j;
      const bool take = t < mm && (select_key(order_key(s[j]), (int32_t)(t0 + t)) & mask) >= prefix;
      sel |= (take ? 1u : 0u) << j;
    }
  }
  int tot;
  int pos = block_exclusive_sum<kSmallThreads>(__popc(sel), wsum, &tot);
  if (!(kk > 0 && t0 < n)) base = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (sel & (1u << j)) {
      if (base + pos < kk) list[pos] = (uint16_t)(tb + j);
      ++pos;
    }
  if (tid == 0) *s_nsel = (int)max<int64_t>(0, min<int64_t>(tot, kk - base));
}

// One step of a recursive-halving sum across the lanes that differ in bit MSK: of a[0, N) a lane
// keeps the half selected by its bit, receives the other half from its partner, and leaves the
// sums in a[0, N/2) (every index is a compile-time constant, so a[] stays in registers).
template <int N, int MSK, int NA>
__device__ __forceinline__ void halve_step(float (&a)[NA], int lane) {
  constexpr int half = N / 2;
  const bool up = (lane & MSK) != 0;
#pragma unroll
  for (int j = 0; j < half; ++j) {
    const float send = up ? a[j] : a[half + j];
    const float keep = up ? a[half + j] : a[j];
    a[j] = keep + __shfl_xor(send, MSK);
  }
}

// Sparse attention, lean form: one query head per KV head, 4-bit key and value codes, no sketch
// (the Self-Indexing layout: the selection does the coarse work, the payload is codes only).
// Four threads per selected token, thread (t, s) owning coordinates [s D/4, (s+1) D/4): it loads
// its slices of the token's key and value fields and the norms straight from the record (three
// independent loads), forms its part of <q_x, gamma[c]> from the level table in LDS, and after
// a quad sum and the batch's softmax keeps w gamma_v[c] in D/4 per-thread accumulators (rescaled
// when the running maximum rises).  At the end the 64 token slots are summed: recursive halving
// across the 16 lanes of a wave that share s, then the four waves through LDS.
template <int D>
__global__ __launch_bounds__(kSmallThreads) void sparse_attend_lean_kernel(SparseArgs S) {
  const DecodeArgs& A = S.a;
  constexpr int QW = D / 4;                 // coordinates per thread
  constexpr int NW = QW / 8;                // 32-bit words of 4-bit codes per thread
  constexpr int TPB = kSmallThreads / 4;    // tokens per batch
  constexpr int OUT = QW / 16;              // coordinates per lane after the in-wave reduction
  using Slice = typename std::conditional<NW == 4, uint4, uint2>::type;
  __shared__ uint16_t list[kSelChunk];
  __shared__ int wsum[kSmallThreads / 64];
  __shared__ int s_nsel;
  __shared__ float kl[16], vl[16];
  __shared__ float red[2][kSmallThreads / 64];
  __shared__ float osum[kSmallThreads / 64][D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int64_t unit = (int64_t)b * A.kv_heads + hkv;
  const int64_t qrow = (int64_t)b * A.q_heads + hkv;
  const int64_t n = min((int64_t)A.seq_lens[b], A.capacity);
  const int64_t kk = min((int64_t)S.k, n);
  const int64_t t0 = (int64_t)c * kSelChunk;
  sparse_chunk_list(S, unit, c, n, kk, list, wsum, &s_nsel);
  if (tid < 16) {
    kl[tid] = A.key_levels[tid];
    vl[tid] = A.val_levels[tid];
  }
  const int sq = tid & 3, tq = tid >> 2;
  float q[QW];
#pragma unroll
  for (int j = 0; j < QW; j += 4) {
    const float4 v = *reinterpret_cast<const float4*>(A.qx + qrow * D + sq * QW + j);
    q[j] = v.x; q[j + 1] = v.y; q[j + 2] = v.z; q[j + 3] = v.w;
  }
  float acc[QW];
#pragma unroll
  for (int j = 0; j < QW; ++j) acc[j] = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;
  __syncthreads();
  const int nsel = s_nsel;
  const uint8_t* recs = A.records + unit * A.capacity * A.rec_bytes;
  const float lscale = A.scale * A.inv_sqrt_d;
  for (int s0 = 0; s0 < nsel; s0 += TPB) {
    const int nt = min(TPB, nsel - s0);
    const bool live = tq < nt;
    const uint8_t* rec = recs + (t0 + list[s0 + min(tq, nt - 1)]) * A.rec_bytes;   // clamped
    const Slice kw = *reinterpret_cast<const Slice*>(rec + sq * (QW / 2));
    const Slice vw = *reinterpret_cast<const Slice*>(rec + A.kbytes + A.sbytes + sq * (QW / 2));
    const float r_k = *reinterpret_cast<const float*>(rec + A.norm_off);
    const float r_v = *reinterpret_cast<const float*>(rec + A.norm_off + 8);
    uint32_t kwv[NW], vwv[NW];
    if constexpr (NW == 4) {
      kwv[0] = kw.x; kwv[1] = kw.y; kwv[2] = kw.z; kwv[3] = kw.w;
      vwv[0] = vw.x; vwv[1] = vw.y; vwv[2] = vw.z; vwv[3] = vw.w;
    } else {
      kwv[0] = kw.x; kwv[1] = kw.y;
      vwv[0] = vw.x; vwv[1] = vw.y;
    }
    // code j of the slice: bits [4 j, 4 j + 4) of the little-endian word stream
    float dot = 0.0f;
#pragma unroll
    for (int wi = 0; wi < NW; ++wi)
#pragma unroll
      for (int u = 0; u < 8; ++u) dot = fmaf(q[8 * wi + u], kl[(kwv[wi] >> (4 * u)) & 15u], dot);
    dot += __shfl_xor(dot, 1);
    dot += __shfl_xor(dot, 2);
    const float lg = live ? lscale * (r_k * dot) : kNegInf;
    float bm = lg;
#pragma unroll
    for (int msk = 4; msk < 64; msk <<= 1) bm = fmaxf(bm, __shfl_xor(bm, msk));
    if (lane == 0) red[0][wave] = bm;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kSmallThreads / 64; ++w) bm = fmaxf(bm, red[0][w]);
    const float mn = fmaxf(m_run, bm);
    const float f = m_run == kNegInf ? 0.0f : __expf(m_run - mn);
    const float p = live ? __expf(lg - mn) : 0.0f;
    float ps = sq == 0 ? p : 0.0f;
#pragma unroll
    for (int msk = 4; msk < 64; msk <<= 1) ps += __shfl_xor(ps, msk);
    if (lane == 0) red[1][wave] = ps;
    __syncthreads();
    float bsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kSmallThreads / 64; ++w) bsum += red[1][w];
    l_run = l_run * f + bsum;
    m_run = mn;
    const float wt = p * r_v * A.inv_sqrt_d;
#pragma unroll
    for (int wi = 0; wi < NW; ++wi)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        acc[8 * wi + u] = fmaf(wt, vl[(vwv[wi] >> (4 * u)) & 15u], acc[8 * wi + u] * f);
    __syncthreads();            // red[] is rewritten by the next batch
  }
  // sum the 16 token slots of this wave that share sq: recursive halving over lane bits 5..2;
  // lane (t', sq) then holds coordinates sq QW + OUT t' + [0, OUT)
  halve_step<QW, 32>(acc, lane);
  halve_step<QW / 2, 16>(acc, lane);
  halve_step<QW / 4, 8>(acc, lane);
  halve_step<QW / 8, 4>(acc, lane);
  const int tl = lane >> 2;
#pragma unroll
  for (int e = 0; e < OUT; ++e) osum[wave][sq * QW + OUT * tl + e] = acc[e];
  __syncthreads();
  const int stride = D + 2;
  float* part = A.part + (qrow * A.n_chunks + c) * stride;
  for (int i = tid; i < D; i += kSmallThreads) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kSmallThreads / 64; ++w) v += osum[w][i];
    part[2 + i] = v;
  }
  if (tid == 0) {
    part[0] = m_run;
    part[1] = l_run;
  }
}

// POLAR: polar key codes; each token's unit vector u is rebuilt into LDS (float32, one thread
// per (token, level-1 pair): the root-first product of the cos / sin factors on its path) and
// the key part of the estimate is r_k <q_x, u>.
template <int D, int BK, int BV, int MG, bool POLAR = false>
__global__ __launch_bounds__(kSmallThreads) void sparse_attend_kernel(SparseArgs S) {
  const DecodeArgs& A = S.a;
  constexpr int NG32 = D / 32, TB = kSmallMaxTok;
  constexpr int KRW = POLAR ? 16 : 1;              // polar key field words per token (at most 64 bytes)
  __shared__ uint32_t kraw[POLAR ? TB : 1][KRW];
  __shared__ float ku[POLAR ? TB : 1][POLAR ? D + 1 : 1];
  __shared__ uint16_t list[kSelChunk];             // selected tokens, offsets within the chunk
  __shared__ int wsum[kSmallThreads / 64];
  __shared__ int s_nsel;
  __shared__ float qx[MG][D + 1];
  __shared__ float qs[MG][kSmallMaxM + 1];
  __shared__ __attribute__((aligned(4))) uint8_t kc[TB][D];
  __shared__ __attribute__((aligned(4))) uint8_t vc[TB][D];
  __shared__ __attribute__((aligned(4))) uint8_t sb[TB][kSmallMaxM];
  __shared__ float nr[TB][3];
  __shared__ float lg[MG][TB + 1];
  __shared__ float hm[MG], hl[MG], hf[MG];
  __shared__ float kl[kMaxLevels], vl[kMaxLevels];
  const int G = A.G, m = A.m, tid = threadIdx.x;
  const int c = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int64_t unit = (int64_t)b * A.kv_heads + hkv;
  const int64_t qrow0 = (int64_t)b * A.q_heads + (int64_t)hkv * G;
  const int64_t n = min((int64_t)A.seq_lens[b], A.capacity);
  const int64_t kk = min((int64_t)S.k, n);
  const int64_t t0 = (int64_t)c * kSelChunk;
  sparse_chunk_list(S, unit, c, n, kk, list, wsum, &s_nsel);
  for (int e = tid; e < G * D; e += kSmallThreads) qx[e / D][e % D] = A.qx[(qrow0 + e / D) * D + e % D];
  for (int e = tid; e < G * m; e += kSmallThreads) qs[e / m][e % m] = A.qs[(qrow0 + e / m) * m + e % m];
  if (tid < kMaxLevels) {
    kl[tid] = A.key_levels[tid];
    vl[tid] = A.val_levels[tid];
  }
  if (tid < G) {
    hm[tid] = kNegInf;
    hl[tid] = 0.0f;
  }
  constexpr int kMaxOut = (MG * D + kSmallThreads - 1) / kSmallThreads;
  float o[kMaxOut];
#pragma unroll
  for (int r = 0; r < kMaxOut; ++r) o[r] = 0.0f;
  __syncthreads();
  const int nsel = s_nsel;
  // SP adjacent threads per (head, coordinate) output when the outputs are fewer than the
  // threads (each sums every SP-th token; the SP partial sums are added at the end)
  int SP = 1;
  while (SP < 4 && G * D * SP * 2 <= kSmallThreads) SP *= 2;
  const uint8_t* recs = A.records + unit * A.capacity * A.rec_bytes;
  const int nsw = m / 32, per_t = 2 * NG32 + nsw + 1;
  for (int s0 = 0; s0 < nsel; s0 += TB) {
    const int nt = min(TB, nsel - s0);
    for (int e = tid; e < nt * per_t; e += kSmallThreads) {
      const int t = e / per_t, pt = e % per_t;
      const uint8_t* rec = recs + (t0 + list[s0 + t]) * A.rec_bytes;
      if (POLAR && pt < NG32) {
        // the raw key field (level-1 stream, upper-level stream), unpacked below
        const uint32_t* src = reinterpret_cast<const uint32_t*>(rec);
        for (int i = pt; i < A.kbytes / 4; i += NG32) kraw[t][i] = src[i];
      } else if (pt < 2 * NG32) {
        const bool key = pt < NG32;
        const int g = key ? pt : pt - NG32;
        uint32_t w[4];
        const uint32_t* src = reinterpret_cast<const uint32_t*>(
            rec + (key ? g * 4 * BK : A.kbytes + A.sbytes + g * 4 * BV));
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = i < (key ? BK : BV) ? src[i] : 0u;
        uint32_t* dst = reinterpret_cast<uint32_t*>(key ? &kc[t][32 * g] : &vc[t][32 * g]);
        const int nb = key ? BK : BV;
        if (nb == 4) {
          // 4-bit codes: nibble j of the word stream -> byte j (low nibbles, high nibbles, then
          // interleaved by byte permutes)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
            dst[2 * i] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
            dst[2 * i + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
          }
        } else {
#pragma unroll
          for (int j4 = 0; j4 < 8; ++j4) {
            uint32_t word = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int j = 4 * j4 + u;
              const uint32_t code = nb == 3 ? group3_code(w[0], w[1], w[2], j) : field<4>(w, j * nb, nb);
              word |= code << (8 * u);
            }
            dst[j4] = word;
          }
        }
      } else if (pt < 2 * NG32 + nsw) {
        const int wi = pt - 2 * NG32;
        const uint32_t sw = reinterpret_cast<const uint32_t*>(rec + A.kbytes)[wi];
        uint32_t* dst = reinterpret_cast<uint32_t*>(&sb[t][32 * wi]);
#pragma unroll
        for (int j4 = 0; j4 < 8; ++j4) {
          const uint32_t nib = (sw >> (4 * j4)) & 15u;
          dst[j4] = (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
        }
      } else {
        const float* f = reinterpret_cast<const float*>(rec + A.norm_off);
        nr[t][0] = f[0];
        nr[t][1] = f[1];
        nr[t][2] = f[2];
      }
    }
    __syncthreads();
    if constexpr (POLAR) {
      const int np = D / 2, l1w = A.l1_bytes / 4;
      for (int e = tid; e < nt * np; e += kSmallThreads) {
        const int t = e / np, pair = e % np;
        float sc = 1.0f;
        for (int l = A.plevels; l >= 2; --l) {
          const int node = pair >> (l - 1), side = (pair >> (l - 2)) & 1;
          const int idx = (D - (D >> (l - 1)) + node) - D / 2, pos = idx * A.pbh;
          const uint32_t code = (kraw[t][l1w + (pos >> 5)] >> (pos & 31)) & ((1u << A.pbh) - 1u);
          sc *= A.pcs[2 * ((l - 1) * 16 + code) + side];
        }
        const int pos1 = pair * A.pb1;
        const uint32_t c1 = (kraw[t][pos1 >> 5] >> (pos1 & 31)) & ((1u << A.pb1) - 1u);
        ku[t][2 * pair] = sc * A.pcs[2 * c1];
        ku[t][2 * pair + 1] = sc * A.pcs[2 * c1 + 1];
      }
      __syncthreads();
    }
    const int items = nt * G;
    int L = 1;
    while (L < 8 && items * L * 2 <= kSmallThreads) L *= 2;
    for (int i0 = 0; i0 < items; i0 += kSmallThreads / L) {
      const int it = i0 + tid / L, s = tid % L;
      const int t = it / G, h = it % G;
      float dot = 0.0f, qd = 0.0f;
      if (it < items) {
        if constexpr (POLAR)
          for (int i = s; i < D; i += L) dot = fmaf(qx[h][i], ku[t][i], dot);
        else
          for (int i = s; i < D; i += L) dot = fmaf(qx[h][i], kl[kc[t][i]], dot);
        for (int j = s; j < m; j += L) qd += sb[t][j] ? qs[h][j] : -qs[h][j];
      }
      for (int msk = 1; msk < L; msk <<= 1) {
        dot += __shfl_xor(dot, msk);
        qd += __shfl_xor(qd, msk);
      }
      if (it < items && s == 0)
        lg[h][t] = A.scale * fmaf(A.qjl_coef * nr[t][1], qd, nr[t][0] * (POLAR ? 1.0f : A.inv_sqrt_d) * dot);
    }
    __syncthreads();
    // online softmax over this batch: one wave per head, one lane per token
    {
      const int lane = tid & 63, wv = tid >> 6;
      for (int h = wv; h < G; h += kSmallThreads / 64) {
        const float x = lane < nt ? lg[h][lane] : kNegInf;
        float bm = x;
#pragma unroll
        for (int msk = 32; msk > 0; msk >>= 1) bm = fmaxf(bm, __shfl_xor(bm, msk));
        const float mo = hm[h], mn = fmaxf(mo, bm);
        const float p = x == kNegInf ? 0.0f : __expf(x - mn);
        float ps = p;
#pragma unroll
        for (int msk = 32; msk > 0; msk >>= 1) ps += __shfl_xor(ps, msk);
        if (lane < nt) lg[h][lane] = p * nr[lane][2] * A.inv_sqrt_d;
        if (lane == 0) {
          const float f = mo == kNegInf ? 0.0f : __expf(mo - mn);
          hf[h] = f;
          hm[h] = mn;
          hl[h] = hl[h] * f + ps;
        }
      }
    }
    __syncthreads();
    if (SP > 1) {
      const int e = tid / SP, sp = tid % SP;
      if (e < G * D) {
        const int h = e / D, i = e % D;
        float acc = o[0] * hf[h];
        for (int t = sp; t < nt; t += SP) acc = fmaf(lg[h][t], vl[vc[t][i]], acc);
        o[0] = acc;
      }
    } else {
#pragma unroll
      for (int r = 0; r < kMaxOut; ++r) {
        const int e = tid + kSmallThreads * r;
        if (e < G * D) {
          const int h = e / D, i = e % D;
          float acc = o[r] * hf[h];
          for (int t = 0; t < nt; ++t) acc = fmaf(lg[h][t], vl[vc[t][i]], acc);
          o[r] = acc;
        }
      }
    }
    __syncthreads();            // the next batch overwrites the codes and weights
  }
  const int stride = D + 2;
  if (SP > 1) {
    float v = o[0];
    for (int msk = 1; msk < SP; msk <<= 1) v += __shfl_xor(v, msk);
    const int e = tid / SP;
    if (tid % SP == 0 && e < G * D) A.part[((qrow0 + e / D) * A.n_chunks + c) * stride + 2 + e % D] = v;
  } else {
#pragma unroll
    for (int r = 0; r < kMaxOut; ++r) {
      const int e = tid + kSmallThreads * r;
      if (e < G * D) A.part[((qrow0 + e / D) * A.n_chunks + c) * stride + 2 + e % D] = o[r];
    }
  }
  for (int h = tid; h < G; h += kSmallThreads) {
    A.part[((qrow0 + h) * A.n_chunks + c) * stride] = hm[h];
    A.part[((qrow0 + h) * A.n_chunks + c) * stride + 1] = hl[h];
  }
}

// Sparse attention for every other head_dim (scalar key codes): the chunk's selected tokens as
// in the other sparse kernels, taken kDecGenTok at a time with decode_generic_kernel's record
// staging and unpacking (d, code widths and sketch width read at run time), an online softmax
// per head across the batches, and the value sums per (head, coordinate) kept in registers.
__global__ __launch_bounds__(kSmallThreads) void sparse_attend_generic_kernel(SparseArgs S) {
  const DecodeArgs& A = S.a;
  constexpr int TB = kDecGenTok, kMaxOut = kSmallMaxG * kGenMaxD / kSmallThreads;
  __shared__ uint16_t list[kSelChunk];
  __shared__ int wsum[kSmallThreads / 64];
  __shared__ int s_nsel;
  __shared__ float qx[kSmallMaxG][kGenMaxD + 1];
  __shared__ float qs[kSmallMaxG][kDecGenMaxM + 1];
  __shared__ __attribute__((aligned(16))) uint32_t raw[TB][kDecGenMaxRec / 4];
  __shared__ uint8_t kc[TB][kGenMaxD];
  __shared__ uint8_t vc[TB][kGenMaxD];
  __shared__ uint8_t sb[TB][kDecGenMaxM];
  __shared__ float nr[TB][3];
  __shared__ float lg[kSmallMaxG][TB + 1];
  __shared__ float hm[kSmallMaxG], hl[kSmallMaxG], hf[kSmallMaxG];
  __shared__ float kl[kMaxLevels], vl[kMaxLevels];
  const int G = A.G, m = A.m, d = A.d, tid = threadIdx.x;
  const int c = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int64_t unit = (int64_t)b * A.kv_heads + hkv;
  const int64_t qrow0 = (int64_t)b * A.q_heads + (int64_t)hkv * G;
  const int64_t n = min((int64_t)A.seq_lens[b], A.capacity);
  const int64_t kk = min((int64_t)S.k, n);
  const int64_t t0 = (int64_t)c * kSelChunk;
  sparse_chunk_list(S, unit, c, n, kk, list, wsum, &s_nsel);
  for (int e = tid; e < G * d; e += kSmallThreads) qx[e / d][e % d] = A.qx[(qrow0 + e / d) * d + e % d];
  for (int e = tid; e < G * m; e += kSmallThreads) qs[e / m][e % m] = A.qs[(qrow0 + e / m) * m + e % m];
  if (tid < kMaxLevels) {
    kl[tid] = A.key_levels[tid];
    vl[tid] = A.val_levels[tid];
  }
  if (tid < G) {
    hm[tid] = kNegInf;
    hl[tid] = 0.0f;
  }
  float o[kMaxOut];
#pragma unroll
  for (int r = 0; r < kMaxOut; ++r) o[r] = 0.0f;
  __syncthreads();
  const int nsel = s_nsel;
  const uint8_t* recs = A.records + unit * A.capacity * A.rec_bytes;
  const int rw = A.rec_bytes / 4, per_t = 2 * d + m;
  for (int s0 = 0; s0 < nsel; s0 += TB) {
    const int nt = min(TB, nsel - s0);
    for (int e = tid; e < nt * rw; e += kSmallThreads) {
      const int t = e / rw, w = e % rw;
      raw[t][w] = reinterpret_cast<const uint32_t*>(recs + (t0 + list[s0 + t]) * A.rec_bytes)[w];
    }
    __syncthreads();
    for (int e = tid; e < nt * per_t; e += kSmallThreads) {
      const int t = e / per_t, j = e % per_t;
      const uint8_t* r = reinterpret_cast<const uint8_t*>(raw[t]);
      if (j < d) kc[t][j] = (uint8_t)field_code(r, j, A.kb, d);
      else if (j < 2 * d) vc[t][j - d] = (uint8_t)field_code(r + A.kbytes + A.sbytes, j - d, A.vb, d);
      else sb[t][j - 2 * d] = (uint8_t)((r[A.kbytes + ((j - 2 * d) >> 3)] >> ((j - 2 * d) & 7)) & 1u);
    }
    for (int t = tid; t < nt; t += kSmallThreads) {
      const float* f = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(raw[t]) + A.norm_off);
      nr[t][0] = f[0];
      nr[t][1] = f[1];
      nr[t][2] = f[2];
    }
    __syncthreads();
    const int items = nt * G;
    int L = 1;
    while (L < 8 && items * L * 2 <= kSmallThreads) L *= 2;
    for (int i0 = 0; i0 < items; i0 += kSmallThreads / L) {
      const int it = i0 + tid / L, sl = tid % L;
      const int t = it / G, h = it % G;
      float dot = 0.0f, qd = 0.0f;
      if (it < items) {
        for (int i = sl; i < d; i += L) dot = fmaf(qx[h][i], kl[kc[t][i]], dot);
        for (int j = sl; j < m; j += L) qd += sb[t][j] ? qs[h][j] : -qs[h][j];
      }
      for (int msk = 1; msk < L; msk <<= 1) {
        dot += __shfl_xor(dot, msk);
        qd += __shfl_xor(qd, msk);
      }
      if (it < items && sl == 0)
        lg[h][t] = A.scale * fmaf(A.qjl_coef * nr[t][1], qd, nr[t][0] * A.inv_sqrt_d * dot);
    }
    __syncthreads();
    {
      const int lane = tid & 63, wv = tid >> 6;
      for (int h = wv; h < G; h += kSmallThreads / 64) {
        const float x = lane < nt ? lg[h][lane] : kNegInf;
        float bm = x;
#pragma unroll
        for (int msk = 32; msk > 0; msk >>= 1) bm = fmaxf(bm, __shfl_xor(bm, msk));
        const float mo = hm[h], mn = fmaxf(mo, bm);
        const float p = x == kNegInf ? 0.0f : __expf(x - mn);
        float ps = p;
#pragma unroll
        for (int msk = 32; msk > 0; msk >>= 1) ps += __shfl_xor(ps, msk);
        if (lane < nt) lg[h][lane] = p * nr[lane][2] * A.inv_sqrt_d;
        if (lane == 0) {
          const float f = mo == kNegInf ? 0.0f : __expf(mo - mn);
          hf[h] = f;
          hm[h] = mn;
          hl[h] = hl[h] * f + ps;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kMaxOut; ++r) {
      const int e = tid + kSmallThreads * r;
      if (e < G * d) {
        const int h = e / d, i = e % d;
        float acc = o[r] * hf[h];
        for (int t = 0; t < nt; ++t) acc = fmaf(lg[h][t], vl[vc[t][i]], acc);
        o[r] = acc;
      }
    }
    __syncthreads();            // the next batch overwrites the records, codes and weights
  }
  const int stride = d + 2;
#pragma unroll
  for (int r = 0; r < kMaxOut; ++r) {
    const int e = tid + kSmallThreads * r;
    if (e < G * d) A.part[((qrow0 + e / d) * A.n_chunks + c) * stride + 2 + e % d] = o[r];
  }
  for (int h = tid; h < G; h += kSmallThreads) {
    A.part[((qrow0 + h) * A.n_chunks + c) * stride] = hm[h];
    A.part[((qrow0 + h) * A.n_chunks + c) * stride + 1] = hl[h];
  }
}

SparsePlan plan_sparse(const Consts& c, int batch, int q_heads, int kv_heads, int64_t capacity) {
  SparsePlan p;
  p.select = plan_select(c, batch, kv_heads, capacity);
  const size_t rows = (size_t)std::max(batch, 1) * q_heads;
  p.ws_select = 0;
  p.ws_qx = align256(p.select.ws_total);
  p.ws_qs = p.ws_qx + align256(rows * c.d * 4);
  p.ws_part = p.ws_qs + align256(rows * std::max(c.m, 1) * 4);
  p.ws_total = p.ws_part + align256(rows * (size_t)std::max(p.select.n_chunks, 1) * (c.d + 2) * 4);
  return p;
}

template <int D, int MG>
static void launch_sparse_d(const SparseArgs& s, int kb, int vb, bool polar, dim3 grid, size_t dyn, hipStream_t st) {
  if (polar) {
#define TQ_SPP(BV_)                                                                                      \
  if (vb == BV_) {                                                                                       \
    allow_lds(sparse_attend_kernel<D, 4, BV_, MG, true>, dyn);                                           \
    hipLaunchKernelGGL((sparse_attend_kernel<D, 4, BV_, MG, true>), grid, dim3(kSmallThreads), dyn, st, s); \
    return;                                                                                              \
  }
    TQ_SPP(1) TQ_SPP(2) TQ_SPP(3) TQ_SPP(4)
#undef TQ_SPP
    return;
  }
#define TQ_SP(BK_, BV_)                                                                                 \
  if (kb == BK_ && vb == BV_) {                                                                         \
    allow_lds(sparse_attend_kernel<D, BK_, BV_, MG>, dyn);                                              \
    hipLaunchKernelGGL((sparse_attend_kernel<D, BK_, BV_, MG>), grid, dim3(kSmallThreads), dyn, st, s); \
    return;                                                                                             \
  }
  TQ_SP(1, 1) TQ_SP(1, 2) TQ_SP(1, 3) TQ_SP(1, 4) TQ_SP(2, 1) TQ_SP(3, 1) TQ_SP(4, 1)
  TQ_SP(2, 2) TQ_SP(2, 3) TQ_SP(2, 4) TQ_SP(3, 2) TQ_SP(3, 3) TQ_SP(3, 4)
  TQ_SP(4, 2) TQ_SP(4, 3) TQ_SP(4, 4)
#undef TQ_SP
}

hipError_t launch_sparse(const Consts& c, const DevConsts& dc, const SparsePlan& plan, const void* q,
                         tq_dtype q_dt, int batch, int q_heads, int kv_heads, const void* index,
                         const float* codebook, const void* records, int64_t capacity,
                         const int32_t* seq_lens, int k, const void* hot_k, const void* hot_v,
                         tq_dtype hot_dt, const int32_t* hot_lens, int64_t hot_capacity, float scale,
                         float* out, float* lse, void* workspace, hipStream_t stream,
                         const ProfileEvents& ev) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const SelectPlan& sp = plan.select;
  float* qx = reinterpret_cast<float*>(ws + plan.ws_qx);
  float* qs = reinterpret_cast<float*>(ws + plan.ws_qs);
  float* part = reinterpret_cast<float*>(ws + plan.ws_part);
  const int rows = batch * q_heads;
  // the query prep rides in the selection's table launch (which runs when capacity > 0)
  const QueryPrep prep{dc.pi, dc.s, c.m, rows, qx, qs};
  // the attention forms the selection threshold itself (no exact launch)
  hipError_t e = launch_select(c, sp, q, q_dt, batch, q_heads, kv_heads, index, codebook, capacity, seq_lens, k,
                               nullptr, nullptr, nullptr, ws + plan.ws_select, stream, ev, &prep, true);
  if (e != hipSuccess) return e;
  if (capacity <= 0)
    hipLaunchKernelGGL(query_prep_kernel, dim3(rows), dim3(kQueryPrepThreads), 0, stream, dc.pi, dc.s, c.d, c.m, q,
                       q_dt, qx, qs);
  const int n_chunks = std::max(sp.n_chunks, 1);
  const float sc = scale > 0.0f ? scale : c.inv_sqrt_d;
  SparseArgs s;
  DecodeArgs& a = s.a;
  a = DecodeArgs{};
  a.qx = qx;
  a.qs = qs;
  a.records = static_cast<const uint8_t*>(records);
  a.seq_lens = seq_lens;
  a.part = part;
  a.capacity = capacity;
  a.d = c.d;
  a.m = c.m;
  a.kbytes = c.kbytes;
  a.sbytes = c.sbytes;
  a.rec_bytes = c.rec_bytes;
  a.norm_off = c.norm_off;
  a.kb = c.kb;
  a.vb = c.vb;
  a.G = q_heads / kv_heads;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.n_chunks = n_chunks;
  a.scale = sc;
  a.inv_sqrt_d = c.inv_sqrt_d;
  a.qjl_coef = c.qjl_coef;
  for (int i = 0; i < kMaxLevels; ++i) {
    a.key_levels[i] = c.key_levels[i];
    a.val_levels[i] = c.val_levels[i];
  }
  a.pcs = dc.polar.cs32;
  a.pb1 = c.pb1;
  a.pbh = c.pbh;
  a.plevels = c.plevels;
  a.l1_bytes = c.l1_bytes;
  s.scores = reinterpret_cast<const int32_t*>(ws + plan.ws_select + sp.ws_scores);
  s.params = reinterpret_cast<const SelectParams*>(ws + plan.ws_select + sp.ws_params);
  s.chunk_off = reinterpret_cast<const int32_t*>(ws + plan.ws_select + sp.ws_chunk_off);
  s.cand_all = reinterpret_cast<const uint2*>(ws + plan.ws_select + sp.ws_cand);
  s.chunk_cand = reinterpret_cast<const int32_t*>(ws + plan.ws_select + sp.ws_chunk_cand);
  s.chunk_above = reinterpret_cast<const int32_t*>(ws + plan.ws_select + sp.ws_chunk_above);
  s.k = k;
  const dim3 grid((unsigned)n_chunks, kv_heads, batch);
  // query rows held in LDS sized for the group (a smaller footprint keeps more workgroups per CU)
  const int G = q_heads / kv_heads;
  const bool lean = G == 1 && c.m == 0 && c.kb == 4 && c.vb == 4 && !c.polar && (c.d == 128 || c.d == 64);
  const size_t dyn = (size_t)n_chunks * 4;     // the threshold's prefix of candidate counts
  if (c.d != 64 && c.d != 128) {
    allow_lds(sparse_attend_generic_kernel, dyn);
    hipLaunchKernelGGL(sparse_attend_generic_kernel, grid, dim3(kSmallThreads), dyn, stream, s);
  } else if (lean && c.d == 128) {
    allow_lds(sparse_attend_lean_kernel<128>, dyn);
    hipLaunchKernelGGL(sparse_attend_lean_kernel<128>, grid, dim3(kSmallThreads), dyn, stream, s);
  } else if (lean) {
    allow_lds(sparse_attend_lean_kernel<64>, dyn);
    hipLaunchKernelGGL(sparse_attend_lean_kernel<64>, grid, dim3(kSmallThreads), dyn, stream, s);
  } else if (c.d == 128 && G <= 4) launch_sparse_d<128, 4>(s, c.kb, c.vb, c.polar != 0, grid, dyn, stream);
  else if (c.d == 128) launch_sparse_d<128, kSmallMaxG>(s, c.kb, c.vb, c.polar != 0, grid, dyn, stream);
  else if (G <= 4) launch_sparse_d<64, 4>(s, c.kb, c.vb, c.polar != 0, grid, dyn, stream);
  else launch_sparse_d<64, kSmallMaxG>(s, c.kb, c.vb, c.polar != 0, grid, dyn, stream);
  MergeArgs mg{};
  mg.pi_t = dc.pi_t;
  mg.part = part;
  mg.q = q;
  mg.q_dt = q_dt;
  mg.hot_k = hot_k;
  mg.hot_v = hot_v;
  mg.hot_dt = hot_dt;
  mg.hot_lens = hot_lens;
  mg.hot_capacity = hot_capacity;
  mg.out = out;
  mg.lse = lse;
  mg.d = c.d;
  mg.G = q_heads / kv_heads;
  mg.q_heads = q_heads;
  mg.kv_heads = kv_heads;
  mg.n_chunks = n_chunks;
  mg.scale = sc;
  return launch_merge(c, mg, batch, stream);
}

// =========================================================================================
// Bulk scan (TurboQuant page, "Leistung bei der Vektorsuche"): every query of a KV head
// against every record, s = <[q_x ; q_s], [(r_k/sqrt(d)) gamma[c] ; sqrt(pi/2)/m rho (2 bit - 1)]>.
// A block dequantizes 64 records and stages 64 prepared queries in LDS, then each thread
// computes a 4 x 4 tile of scores.
// =========================================================================================
static bool scan_mfma_path(const Consts& c) {
  return !c.polar && c.d == 128 && (c.kb == 2 || c.kb == 3) && (c.m == 0 || c.m == 128);
}

ScanPlan plan_scan(const Consts& c, int batch, int heads, int n_queries) {
  ScanPlan p;
  const size_t units = (size_t)std::max(batch, 1) * heads;
  p.mfma = scan_mfma_path(c);
  // matrix-core path: groups of 4 queries, whole 16-query tiles of them
  p.n_groups = (std::max(n_queries, 1) + 15) / 16 * 4;
  p.ws_q = 0;
  // generic path: fp16 hi and lo query rows [units][nq][kp], then the row scales
  p.kp = (c.d + c.m + 31) / 32 * 32;
  const size_t rows = units * (size_t)std::max(n_queries, 1);
  p.ws_ql = align256(rows * p.kp * 2);
  p.ws_qscale = p.ws_ql + align256(rows * p.kp * 2);
  p.ws_total = p.mfma ? align256(units * (p.n_groups / 4) * kScanChunks * 64 * 16)   // query operands
                      : p.ws_qscale + align256(rows * 4);
  return p;
}

// Generic bulk scan (every shape off the int8 matrix-core path, e.g. head_dim 200): a dense
// contraction over the d + m operands of each (query, vector) pair on fp16 matrix cores.
// Query rows (q_x | q_s) and token rows (r_k/sqrt(d) gamma[c] | +-coef rho) are each scaled by
// their largest |entry| and split into fp16 hi + lo (RNE; x ~ hi + lo to ~2^-23), and the
// products hi.hi + hi.lo + lo.hi (v_mfma_f32_16x16x32_f16) give each estimate to ~2^-22 of
// sum |q_k t_k|; the two scales multiply the result.
// Prep (one block per query row): q_x = Pi q and q_s = S q_x in float64, then the scaled fp16
// hi / lo rows, zero-padded to kp (a multiple of 32), and the row scale.
// The sketch part q_s (about sqrt(d) times the size of q_x's entries) is divided by sfix, a
// power of two near sqrt(d), and the vectors' sign operands are multiplied by it, so both rows
// keep entries of similar size and their fp16 lo halves stay clear of the subnormal range.
constexpr int kScanPrepThreads = 256;   // 1,024 threads per row measured slower (32 against 28 us)
__global__ __launch_bounds__(kScanPrepThreads) void scan_prep_f16_kernel(const float* __restrict__ pi, const float* __restrict__ s,
                                                            int d, int m, int kp, float sfix, const void* q,
                                                            tq_dtype q_dt, uint16_t* qh, uint16_t* ql,
                                                            float* qscale) {
  __shared__ double qv[256];
  __shared__ double xv[256];
  __shared__ float row[512];
  __shared__ float red[kScanPrepThreads / 64];
  const int64_t r = blockIdx.x;
  const int K = d + m;
  for (int i = threadIdx.x; i < d; i += blockDim.x) qv[i] = (double)load_elem(q, q_dt, r * d + i);
  __syncthreads();
  block_gemv_f64(pi, qv, d, d, [&](int i, double y) {
    xv[i] = y;
    row[i] = (float)y;
  });
  __syncthreads();
  block_gemv_f64(s, xv, m, d, [&](int k, double y) { row[d + k] = (float)y / sfix; });
  __syncthreads();
  float mx = 0.0f;
  for (int k = threadIdx.x; k < K; k += blockDim.x) mx = fmaxf(mx, fabsf(row[k]));
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < kScanPrepThreads / 64; ++w) mx = fmaxf(mx, red[w]);
  const float sc = mx > 0.0f ? mx : 1.0f, inv = 1.0f / sc;
  for (int k = threadIdx.x; k < kp; k += blockDim.x) {
    const float v = k < K ? row[k] * inv : 0.0f;
    const _Float16 h = (_Float16)v;
    const _Float16 l = (_Float16)(v - (float)h);
    qh[r * kp + k] = __builtin_bit_cast(uint16_t, h);
    ql[r * kp + k] = __builtin_bit_cast(uint16_t, l);
  }
  if (threadIdx.x == 0) qscale[r] = sc;
}

__device__ __forceinline__ uint32_t key_code_at(const uint32_t* kw, int i, int d, int kb) {
  if (kb == 3) {
    const int ng = d / 32;
    if (i < 32 * ng) {
      const uint32_t* gw = kw + 3 * (i >> 5);
      return group3_code(gw[0], gw[1], gw[2], i & 31);
    }
    const int pos = 96 * ng + 3 * (i - 32 * ng), wi = pos >> 5, sh = pos & 31;
    uint32_t v = kw[wi] >> sh;
    if (sh + 3 > 32) v |= kw[wi + 1] << (32 - sh);
    return v & 7u;
  }
  const int pos = i * kb, wi = pos >> 5, sh = pos & 31;   // 1-, 2-, 4-bit codes never straddle
  return (kw[wi] >> sh) & ((1u << kb) - 1u);
}

constexpr int kS16Tile = 128;   // queries and vectors per workgroup
constexpr int kS16Row = 40;     // LDS row: 32 fp16 of one K step + 8 pad (80 B)
constexpr int kS16OutRow = 68;  // score staging row: 64 floats + 4 pad (16-byte aligned)

struct Scan16Args {
  const uint16_t* qh;
  const uint16_t* ql;
  const float* qscale;
  const uint8_t* records;
  float* scores;
  int64_t capacity, n_tokens;
  int d, m, kp, kb, kbytes, rec_bytes, norm_off, n_queries;
  float inv_sqrt_d, qjl_coef, gmax, sfix;
  float key_levels[kMaxLevels];
  // polar keys: cos / sin of the grids [8][16][2] (float64), code widths, levels, level-1 stream bytes
  const double* pcs;
  int pb1, pbh, plevels, l1_bytes;
};

// 128 queries x 128 vectors per workgroup; wave w computes queries 64 (w / 2) .. + 63 against
// vectors 64 (w % 2) .. + 63 as 4 x 4 tiles of 16 x 16.  Per K step of 32: thread (row
// tid / 2, half tid % 2) stages 16 operands of one query row (copied) and of one vector, then
// every wave reads its A (queries) and B (vectors) hi / lo operands and issues 48 products.
// A vector's scale is r_k/sqrt(d) max|gamma|, so its key operands gamma[c] / max|gamma| are
// per-code constants: pairs of codes index tables of packed fp16 hi (and lo) pairs.  Its sign
// operands are +-coef rho / scale: one fp16 hi / lo pair per vector, the sign bit flipped by
// the QJL bit.
// POLAR: a vector's scale is r_k and its key operands are the unit vector u of its grid
// angles; the thread staging 16 coordinates (the subtree of one level-4 node) takes the
// subtree root's scale from its ancestors' cos / sin and rebuilds the 16 coordinates top-down
// in float64 (unscaled estimates carry r_k |q|, so float32 products of up to seven table
// entries would cost ~1e-4 absolute), rounded once to float32 before the split.
template <bool POLAR>
__global__ __launch_bounds__(256, 2) void scan_mfma16_kernel(Scan16Args A) {
  // operand staging; after the last K step each wave's 32 x 64 score halves (the stores' staging)
  __shared__ __attribute__((aligned(16))) union {
    struct {
      uint16_t q[2][kS16Tile * kS16Row];
      uint16_t t[2][kS16Tile * kS16Row];
    } op;
    float out[4][32][kS16OutRow];
  } s16;
  uint16_t (&sq)[2][kS16Tile * kS16Row] = s16.op.q;
  uint16_t (&st)[2][kS16Tile * kS16Row] = s16.op.t;
  __shared__ float sts[kS16Tile];
  __shared__ uint32_t ptab[2][256];    // code pair (c0 | c1 << kb) -> packed fp16 hi / lo pair
  __shared__ double2 pcs[POLAR ? kMaxPolarLevels * 16 : 1];
  if (POLAR && threadIdx.x < kMaxPolarLevels * 16)
    pcs[threadIdx.x] = make_double2(A.pcs[2 * threadIdx.x], A.pcs[2 * threadIdx.x + 1]);
  const int unit = blockIdx.z;
  const int64_t t0 = (int64_t)blockIdx.x * kS16Tile;
  const int q0 = blockIdx.y * kS16Tile;
  const int K = A.d + A.m, kb = A.kb;
  const float ginv = A.gmax > 0.0f ? 1.0f / A.gmax : 0.0f;
  for (int e = threadIdx.x; e < (1 << (2 * kb)); e += blockDim.x) {
    uint32_t hp = 0u, lp = 0u;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float v = A.key_levels[(e >> (kb * u)) & ((1 << kb) - 1)] * ginv;
      const _Float16 h = (_Float16)v;
      const _Float16 l = (_Float16)(v - (float)h);
      hp |= (uint32_t)__builtin_bit_cast(uint16_t, h) << (16 * u);
      lp |= (uint32_t)__builtin_bit_cast(uint16_t, l) << (16 * u);
    }
    ptab[0][e] = hp;
    ptab[1][e] = lp;
  }
  // staging role
  const int ri = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int64_t t = t0 + ri;
  const bool tv = t < A.n_tokens;
  const uint8_t* rec = A.records + ((int64_t)unit * A.capacity + (tv ? t : 0)) * A.rec_bytes;
  const float* nrm = reinterpret_cast<const float*>(rec + A.norm_off);
  const float ak = tv ? nrm[0] * A.inv_sqrt_d : 0.0f, aq = tv ? A.qjl_coef * nrm[1] : 0.0f;
  const float tsc = POLAR ? (tv ? nrm[0] : 0.0f) : ak * A.gmax;   // 0 for an invalid or zero vector (then aq = 0)
  const float sv = tsc > 0.0f ? aq * A.sfix / tsc : 0.0f;
  uint32_t sgh, sgl;                                   // +sv as an fp16 hi / lo pair in both halves
  {
    const _Float16 h = (_Float16)sv;
    const _Float16 l = (_Float16)(sv - (float)h);
    sgh = (uint32_t)__builtin_bit_cast(uint16_t, h) * 0x10001u;
    sgl = (uint32_t)__builtin_bit_cast(uint16_t, l) * 0x10001u;
  }
  if (half == 0) sts[ri] = tsc;
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(rec);
  const uint32_t* sw = reinterpret_cast<const uint32_t*>(rec + A.kbytes);
  const int qi = q0 + ri;
  const bool qv = qi < A.n_queries;
  const int64_t qrow = ((int64_t)unit * A.n_queries + (qv ? qi : 0)) * A.kp;
  // compute role
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int qb = (wave >> 1) * 64, tb = (wave & 1) * 64;
  f32x4 acc[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  __syncthreads();   // ptab
  for (int k0 = 0; k0 < A.kp; k0 += 32) {
    {
      const int c0 = k0 + 16 * half;
      u32x4 h0 = u32x4{0u, 0u, 0u, 0u}, h1 = h0, l0 = h0, l1 = h0;
      if (qv) {
        const u32x4* ph = reinterpret_cast<const u32x4*>(A.qh + qrow + c0);
        const u32x4* pl = reinterpret_cast<const u32x4*>(A.ql + qrow + c0);
        h0 = ph[0];
        h1 = ph[1];
        l0 = pl[0];
        l1 = pl[1];
      }
      u32x4* dh = reinterpret_cast<u32x4*>(&sq[0][ri * kS16Row + 16 * half]);
      u32x4* dl = reinterpret_cast<u32x4*>(&sq[1][ri * kS16Row + 16 * half]);
      dh[0] = h0;
      dh[1] = h1;
      dl[0] = l0;
      dl[1] = l1;
      // 8 operand pairs (c0 + 2 e2, + 1); d and K are even, so a pair never mixes regions
      uint32_t hw[8], lw[8];
      float pu[16];                                   // polar: the subtree's unit-vector coordinates
      if (POLAR && c0 < A.d) {
        const int bh = A.pbh, b1 = A.pb1, d = A.d;
        const uint32_t mh = (1u << bh) - 1u;
        auto up_code = [&](int l, int node) -> uint32_t {
          const int bit = (d / 2 - (d >> (l - 1)) + node) * bh;
          return (*reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(kw) + A.l1_bytes +
                                                     4 * (bit >> 5)) >> (bit & 31)) & mh;
        };
        double sc = 1.0;
#pragma unroll
        for (int l = kMaxPolarLevels - 1; l >= 5; --l) {
          if (l <= A.plevels) {
            const double2 tc = pcs[(l - 1) * 16 + up_code(l, c0 >> l)];
            sc *= ((c0 >> (l - 1)) & 1) ? tc.y : tc.x;
          }
        }
        double s3[2], s2[4], s1[8];
        {
          const double2 tc = pcs[3 * 16 + up_code(4, c0 >> 4)];
          s3[0] = sc * tc.x;
          s3[1] = sc * tc.y;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const double2 tc = pcs[2 * 16 + up_code(3, (c0 >> 3) + i)];
          s2[2 * i] = s3[i] * tc.x;
          s2[2 * i + 1] = s3[i] * tc.y;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const double2 tc = pcs[16 + up_code(2, (c0 >> 2) + i)];
          s1[2 * i] = s2[i] * tc.x;
          s1[2 * i + 1] = s2[i] * tc.y;
        }
        const int b0 = (c0 >> 1) * b1;                // the 8 level-1 codes: one run of 16 or 32 bits
        const uint32_t w1 = kw[b0 >> 5] >> (b0 & 31);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double2 tc = pcs[(w1 >> (b1 * i)) & ((1u << b1) - 1u)];
          pu[2 * i] = (float)(s1[i] * tc.x);
          pu[2 * i + 1] = (float)(s1[i] * tc.y);
        }
      }
      const bool plain = kb != 3 && c0 + 16 <= A.d;   // 16 key codes of 1, 2 or 4 bits: one run of bits
      uint32_t kr0 = 0u, kr1 = 0u;
      if (plain) {
        const int bit = c0 * kb;
        kr0 = kw[bit >> 5] >> (bit & 31);
        kr1 = kb == 4 ? kw[(bit >> 5) + 1] : 0u;
      }
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {
        const int k = c0 + 2 * e2;
        uint32_t hp = 0u, lp = 0u;
        if (POLAR && k < A.d) {
          const float v0 = pu[2 * e2], v1 = pu[2 * e2 + 1];
          const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
          const _Float16 r0 = (_Float16)(v0 - (float)h0), r1 = (_Float16)(v1 - (float)h1);
          hp = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
          lp = (uint32_t)__builtin_bit_cast(uint16_t, r0) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16);
        } else if (k < A.d) {
          uint32_t pidx;
          if (plain) {
            const int sh = 2 * kb * e2;                 // < 32 for kb = 1, 2; kb = 4: words of 4 pairs
            pidx = kb == 4 ? ((e2 < 4 ? kr0 : kr1) >> (8 * (e2 & 3))) & 0xFFu
                           : (kr0 >> sh) & ((1u << (2 * kb)) - 1u);
          } else {
            pidx = key_code_at(kw, k, A.d, kb) | (key_code_at(kw, k + 1, A.d, kb) << kb);
          }
          hp = ptab[0][pidx];
          lp = ptab[1][pidx];
        } else if (k < K) {
          const int j = k - A.d;
          const uint32_t b2 = (sw[j >> 5] >> (j & 31)) & 3u;
          const uint32_t neg = ((b2 & 1u) ? 0u : 0x8000u) | ((b2 & 2u) ? 0u : 0x80000000u);
          hp = sgh ^ neg;
          lp = sgl ^ neg;
        }
        hw[e2] = hp;
        lw[e2] = lp;
      }
      u32x4* th = reinterpret_cast<u32x4*>(&st[0][ri * kS16Row + 16 * half]);
      u32x4* tl = reinterpret_cast<u32x4*>(&st[1][ri * kS16Row + 16 * half]);
      th[0] = u32x4{hw[0], hw[1], hw[2], hw[3]};
      th[1] = u32x4{hw[4], hw[5], hw[6], hw[7]};
      tl[0] = u32x4{lw[0], lw[1], lw[2], lw[3]};
      tl[1] = u32x4{lw[4], lw[5], lw[6], lw[7]};
    }
    __syncthreads();
    f16x8 ah[4], al[4], bh[4], bl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ah[i] = *reinterpret_cast<const f16x8*>(&sq[0][(qb + 16 * i + n) * kS16Row + 8 * kg]);
      al[i] = *reinterpret_cast<const f16x8*>(&sq[1][(qb + 16 * i + n) * kS16Row + 8 * kg]);
      bh[i] = *reinterpret_cast<const f16x8*>(&st[0][(tb + 16 * i + n) * kS16Row + 8 * kg]);
      bl[i] = *reinterpret_cast<const f16x8*>(&st[1][(tb + 16 * i + n) * kS16Row + 8 * kg]);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt], bh[ct], acc[rt][ct], 0, 0, 0);
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt], bl[ct], acc[rt][ct], 0, 0, 0);
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[rt], bh[ct], acc[rt][ct], 0, 0, 0);
      }
    __syncthreads();   // the next step restages sq / st
  }
  // lane (n, kg) of tile (rt, ct) holds query qb + 16 rt + 4 kg + r against vector tb + 16 ct + n.
  // The scores go out through the wave's LDS staging, 32 query rows at a time, so that each
  // store writes 4 rows x 256 contiguous bytes instead of 4 rows x 64 bytes.
  const bool vec = A.n_tokens % 4 == 0 && reinterpret_cast<uintptr_t>(A.scores) % 16 == 0;
  float (*so)[kS16OutRow] = s16.out[wave];
#pragma unroll
  for (int hr = 0; hr < 2; ++hr) {
#pragma unroll
    for (int rt2 = 0; rt2 < 2; ++rt2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rt2 + 4 * kg + r, qq = q0 + qb + 32 * hr + row;
        const float qs = qq < A.n_queries ? A.qscale[(int64_t)unit * A.n_queries + qq] : 0.0f;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          so[row][16 * ct + n] = acc[2 * hr + rt2][ct][r] * qs * sts[tb + 16 * ct + n];
      }
    wave_lds_sync();
    const int col = 4 * (lane & 15);
    const int64_t tok = t0 + tb + col;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = (lane >> 4) + 4 * j, qq = q0 + qb + 32 * hr + row;
      if (qq >= A.n_queries) continue;
      const float4 v = *reinterpret_cast<const float4*>(&so[row][col]);
      float* o = A.scores + ((int64_t)unit * A.n_queries + qq) * A.n_tokens + tok;
      if (vec && tok + 3 < A.n_tokens) {
        nt_store4(o, f32x4{v.x, v.y, v.z, v.w});
      } else {
        if (tok < A.n_tokens) o[0] = v.x;
        if (tok + 1 < A.n_tokens) o[1] = v.y;
        if (tok + 2 < A.n_tokens) o[2] = v.z;
        if (tok + 3 < A.n_tokens) o[3] = v.w;
      }
    }
    wave_lds_sync();   // the second half's writes follow these reads
  }
}

// -----------------------------------------------------------------------------------------
// Matrix-core bulk scan (head_dim 128, 2- or 3-bit keys, m in {0, 128}): the decode's exact
// int32 estimator over tiles of 16 tokens x 16 queries.  A = token operands (rows = 16 tokens:
// key level limbs by v_perm_b32 from one table per limb plane, QJL bits as 0/1 bytes), B = query
// operands (columns = 16 queries: the int8 limbs of the fixed-point q_x and q_s from
// mfma_prep_kernel in SCAN mode), one int32 accumulator per weight class.  Unscaled estimates
// carry the key norm's full size, so the levels take three int8 limbs here (24 bits,
// F_k = 127 * 65536 / max |level|).  With level limb b and query limb a the key products of
// weight 2^(8 (a + b)) go to class e = 4 - a - b; classes 0..3 are kept (1, 2, 3 and 2 limb
// pairs over two 64-wide K chunks: 16 MFMAs), class 4 (2^0) is dropped; the sketch takes its
// three query limbs against the bits (6 MFMAs).  Lane (query column n, K slice kg) ends with
// tokens 4 kg .. 4 kg + 3 of the tile for query n and writes them with one 16-byte store:
//   s = (r_k/sqrt(d)) ((256 C0 + C1) 2^24 + (256 C2 + C3) 2^8) / (F_q F_k)
//     + coef rho ((2^16 Cq0 + 2^8 Cq1 + Cq2) 2 / F_s - sum / F_s).
// (|C0| < 2^21, |C1| < 2^22, |C2| < 2^23, |C3| < 2^22 and the sketch classes fit the int32
// pair sums.)  A workgroup holds 4 query tiles (64 queries, 13 x 16 B per lane and tile) in
// LDS; each wave walks 32-token steps of a 1024-token range, building two token tiles'
// operands once per step and sweeping the query tiles over them.
// -----------------------------------------------------------------------------------------
constexpr int kScanQT = 4;                  // 16-query tiles per workgroup
constexpr int kScanQB = 16 * kScanQT;       // queries per workgroup
constexpr int kScanTT = 2;                  // 16-token tiles per wave step
constexpr int kScanWaves = 4;               // waves per workgroup
constexpr int kScanThreads = 64 * kScanWaves;
constexpr int kScanBlockTok = 1024;         // tokens per workgroup

struct ScanMfmaArgs {
  const u32x4* qop;        // [unit][query tile][chunk][lane]
  const uint8_t* records;
  float* scores;
  int64_t capacity, n_tokens;
  int rec_bytes, kbytes, norm_off, n_queries, n_qtiles, vec_store;
  float inv_sqrt_d, qjl_coef, key_fix3;
  float key_levels[kMaxLevels];
};

// after the query operands: each wave's 16-query x 32-token score staging (rows padded to 36
// floats, 16-byte aligned)
constexpr int kScanStgRow = 36;
constexpr size_t kScanLds = (size_t)kScanQT * kScanChunks * 64 * 16 + (size_t)kScanWaves * 16 * kScanStgRow * 4;

template <int BK, bool QJL>
__global__ __launch_bounds__(kScanThreads, 2) void scan_mfma_kernel(ScanMfmaArgs A) {
  constexpr int TT = kScanTT;
  extern __shared__ u32x4 qop_lds[];                   // [query tile][chunk][lane]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int unit = blockIdx.z, qb = blockIdx.y;
  const int n = lane & 15, kg = lane >> 4;
  const int qt_end = min(kScanQT, A.n_qtiles - qb * kScanQT);   // query tiles present
  {
    const u32x4* src = A.qop + ((int64_t)unit * A.n_qtiles + qb * kScanQT) * kScanChunks * 64;
    for (int e = threadIdx.x; e < qt_end * kScanChunks * 64; e += kScanThreads) qop_lds[e] = src[e];
  }
  // key levels as three int8 limbs: gamma ~= (65536 l2 + 256 l1 + l0) / F_k; byte c of each
  // table word = code c, one table per limb plane
  const float fk = A.key_fix3;
  uint32_t tp[3][2] = {{0, 0}, {0, 0}, {0, 0}};
#pragma unroll
  for (int c = 0; c < (1 << BK); ++c) {
    int l2, l1, l0;
    int8_limbs3((int)rintf(A.key_levels[c] * fk), l2, l1, l0);
    tp[2][c >> 2] |= (uint32_t)(l2 & 0xFF) << (8 * (c & 3));
    tp[1][c >> 2] |= (uint32_t)(l1 & 0xFF) << (8 * (c & 3));
    tp[0][c >> 2] |= (uint32_t)(l0 & 0xFF) << (8 * (c & 3));
  }
  __syncthreads();

  const uint8_t* recs = A.records + (int64_t)unit * A.capacity * A.rec_bytes;
  const int64_t tlast = A.n_tokens - 1;
  const size_t kofs = (size_t)kg * 4 * BK, sofs = (size_t)A.kbytes + 4 * kg, nofs = (size_t)A.norm_off;
  // lane (row n, K slice kg) of token tile tt reads token 16 tt + n's key words of slice kg,
  // its sketch word and its two norms
  struct Raw {
    uint32_t kw[TT][BK];
    uint32_t sw[TT];
    float2 nrm[TT];
  };
  auto fetch = [&](int64_t t0, Raw& r) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const uint8_t* rec = recs + (size_t)min(t0 + 16 * tt + n, tlast) * A.rec_bytes;
      if constexpr (BK == 3) {
        typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
        const u32x3 w = *reinterpret_cast<const u32x3*>(rec + kofs);
        r.kw[tt][0] = w[0];
        r.kw[tt][BK > 1 ? 1 : 0] = w[1];
        r.kw[tt][BK > 2 ? 2 : 0] = w[2];
      } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(rec + kofs);
        r.kw[tt][0] = w[0];
        r.kw[tt][BK > 1 ? 1 : 0] = w[1];
      }
      r.sw[tt] = QJL ? *reinterpret_cast<const uint32_t*>(rec + sofs) : 0u;
      const float* nrm = reinterpret_cast<const float*>(rec + nofs);
      r.nrm[tt] = make_float2(nrm[0], nrm[1]);
    }
  };
  const int64_t tb0 = (int64_t)blockIdx.x * kScanBlockTok;
  const int64_t tb1 = min(A.n_tokens, tb0 + kScanBlockTok);
  constexpr int kStep = 16 * TT;
  // one step: the token tiles' operands from the raw words, then every query tile against them
  auto step = [&](int64_t t0, const Raw& cur, auto full_tag) {
    // token operands of the tiles: Tk[tt][2 pb + hh] = level limb plane 2 - pb, K chunk hh
    i32x4 Tk[TT][6], Ts[TT][2];
    // scales of the lane's output tokens 16 tt + 4 kg + r, fetched by lane (4 kg + r, any slice)
    float ak[TT][4], aq[TT][4];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      uint32_t sel[8];
      if constexpr (BK == 3) {
        const uint32_t top = group3_top(cur.kw[tt][0], cur.kw[tt][1], cur.kw[tt][2]);
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          sel[2 * s] = cur.kw[tt][s] & 0x07070707u;
          sel[2 * s + 1] = (cur.kw[tt][s] >> 3) & 0x07070707u;
        }
        sel[6] = top & 0x07070707u;
        sel[7] = (top >> 3) & 0x07070707u;
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) sel[s] = (cur.kw[tt][s >> 2] >> (2 * (s & 3))) & 0x03030303u;
      }
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        const int plane = 2 - (j >> 1), hh = j & 1;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          Tk[tt][j][w] = (int)__builtin_amdgcn_perm(tp[plane][1], tp[plane][0], sel[4 * hh + w]);
      }
      if (QJL)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int w = 0; w < 4; ++w) Ts[tt][jj][w] = (int)((cur.sw[tt] >> (4 * jj + w)) & 0x01010101u);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ak[tt][r] = __shfl(cur.nrm[tt].x, 4 * kg + r) * A.inv_sqrt_d;
        aq[tt][r] = QJL ? A.qjl_coef * __shfl(cur.nrm[tt].y, 4 * kg + r) : 0.0f;
      }
    }
    // one query tile against the step's token tiles; FULL: every query and token of the step
    // is present and rows take 16-byte stores, so the tile's code has no branch
    auto qtile = [&](int qt, auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      const u32x4* qo = qop_lds + qt * kScanChunks * 64 + lane;
      i32x4 Q[6], S[6];
#pragma unroll
      for (int c = 0; c < 6; ++c) Q[c] = __builtin_bit_cast(i32x4, qo[c * 64]);
      if (QJL)
#pragma unroll
        for (int c = 0; c < 6; ++c) S[c] = __builtin_bit_cast(i32x4, qo[(6 + c) * 64]);
      const u32x4 scw = qo[12 * 64];
      const float bk = __uint_as_float(scw[0]), bq = __uint_as_float(scw[1]), oq = __uint_as_float(scw[2]);
      const float sk_hi = 16777216.0f * bk, sk_lo = 256.0f * bk;
      i32x4 C[4][TT], Cq[3][TT];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) C[e][tt] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 3; ++e)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) Cq[e][tt] = i32x4{0, 0, 0, 0};
      // level plane 2 - pb against query limb 2 - bi: class pb + bi (kept while <= 3)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int pb = 0; pb < 3; ++pb)
#pragma unroll
          for (int bi = 0; bi < 3; ++bi)
            if (pb + bi <= 3)
#pragma unroll
              for (int tt = 0; tt < TT; ++tt)
                C[pb + bi][tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Tk[tt][2 * pb + hh], Q[2 * bi + hh], C[pb + bi][tt], 0, 0, 0);
      if (QJL)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int bi = 0; bi < 3; ++bi)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
              Cq[bi][tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Ts[tt][jj], S[2 * bi + jj], Cq[bi][tt], 0, 0, 0);
      const int q = qb * kScanQB + 16 * qt + n;
      if (!FULL && q >= A.n_queries) return;
      float* o = A.scores + ((int64_t)unit * A.n_queries + q) * A.n_tokens;
      // FULL: the tile's 16 x 32 scores go through the wave's LDS staging, so that each store
      // writes 8 rows x 128 contiguous bytes (whole lines) instead of 16 rows x 64 bytes
      float* stg = reinterpret_cast<float*>(qop_lds + kScanQT * kScanChunks * 64) + wave * 16 * kScanStgRow;
      if (FULL) wave_lds_sync();   // the previous tile's staging reads are done
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        float sv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float key = fmaf((float)((C[0][tt][r] << 8) + C[1][tt][r]), sk_hi,
                                 (float)((C[2][tt][r] << 8) + C[3][tt][r]) * sk_lo);
          float s = ak[tt][r] * key;
          if (QJL) {
            const float qj = fmaf((float)((((Cq[0][tt][r] << 8) + Cq[1][tt][r]) << 8) + Cq[2][tt][r]), bq, oq);
            s = fmaf(aq[tt][r], qj, s);
          }
          sv[r] = s;
        }
        const int64_t tok = t0 + 16 * tt + 4 * kg;
        if (FULL) {
          *reinterpret_cast<float4*>(stg + n * kScanStgRow + 16 * tt + 4 * kg) = make_float4(sv[0], sv[1], sv[2], sv[3]);
        } else if (A.vec_store && tok + 3 < tb1) {
          *reinterpret_cast<float4*>(o + tok) = make_float4(sv[0], sv[1], sv[2], sv[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (tok + r < tb1) o[tok + r] = sv[r];
        }
      }
      if (FULL) {
        wave_lds_sync();
        // lane L: row 8 i + L / 8 of the tile, tokens 4 (L % 8) .. + 3 of the step
        const int row = lane >> 3, col = 4 * (lane & 7);
        float* orow = A.scores + ((int64_t)unit * A.n_queries + qb * kScanQB + 16 * qt + row) * A.n_tokens + t0 + col;
#pragma unroll
        for (int i = 0; i < 2; ++i)
          nt_store4(orow + (int64_t)8 * i * A.n_tokens, *reinterpret_cast<const f32x4*>(stg + (8 * i + row) * kScanStgRow + col));
      }
    };
    if constexpr (decltype(full_tag)::value) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qt = 0; qt < kScanQT; ++qt) qtile(qt, std::true_type{});
    } else {
      for (int qt = 0; qt < qt_end; ++qt) qtile(qt, std::false_type{});
    }
  };
  int64_t t0 = tb0 + (int64_t)wave * kStep;
  // Workgroups with all their queries present and 16-byte aligned rows run their whole steps
  // branch-free, each fetching the records of the step after it (clamped, so always in
  // bounds) before its own stores, into two register sets used in turn (no copies).  One
  // counter covers loads and stores, and it counts in order: every wait for a step's records
  // finds exactly one step's stores and one step's loads issued after them, so it leaves those
  // in flight.
  if (qt_end == kScanQT && qb * kScanQB + kScanQB <= A.n_queries && A.vec_store) {
    const int64_t t_whole = tb0 + (tb1 - tb0) / kStep * kStep;   // end of the whole steps
    constexpr int64_t kAdv = kScanWaves * kStep;
    if (t0 < t_whole) {
      Raw ra, rb;
      fetch(t0, ra);
      fetch(t0 + kAdv, rb);
      step(t0, ra, std::true_type{});
      t0 += kAdv;
      while (t0 < t_whole) {
        fetch(t0 + kAdv, ra);
        step(t0, rb, std::true_type{});
        t0 += kAdv;
        if (t0 >= t_whole) break;
        fetch(t0 + kAdv, rb);
        step(t0, ra, std::true_type{});
        t0 += kAdv;
      }
    }
  }
  for (; t0 < tb1; t0 += kScanWaves * kStep) {
    Raw cur;
    fetch(t0, cur);
    step(t0, cur, std::false_type{});
  }
}

template <int BK, bool QJL>
static void launch_scan_mfma(dim3 grid, const ScanMfmaArgs& a, hipStream_t stream) {
  allow_lds(scan_mfma_kernel<BK, QJL>, kScanLds);
  hipLaunchKernelGGL((scan_mfma_kernel<BK, QJL>), grid, dim3(kScanThreads), kScanLds, stream, a);
}

hipError_t launch_scan(const Consts& c, const DevConsts& dc, const ScanPlan& plan, const void* q, tq_dtype q_dt,
                       int batch, int heads, int n_queries, const void* records, int64_t capacity,
                       int64_t n_tokens, float* scores, void* workspace, hipStream_t stream,
                       const ProfileEvents& ev) {
  if (plan.mfma) {
    uint32_t* qop = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + plan.ws_q);
    const dim3 pgrid((unsigned)(batch * heads * plan.n_groups));
    const bool qjl = c.m > 0;
    // q viewed as [units][n_queries] rows: "heads" of the prep = queries per unit, groups per unit
    if (c.kb == 3 && qjl)
      hipLaunchKernelGGL((mfma_prep_kernel<3, true, true>), pgrid, dim3(kPrepThreads), 0, stream, dc.pi, dc.s_pi, q, q_dt, n_queries, plan.n_groups, c.key_fix3, qop, nullptr);
    else if (c.kb == 3)
      hipLaunchKernelGGL((mfma_prep_kernel<3, false, true>), pgrid, dim3(kPrepThreads), 0, stream, dc.pi, dc.s_pi, q, q_dt, n_queries, plan.n_groups, c.key_fix3, qop, nullptr);
    else if (qjl)
      hipLaunchKernelGGL((mfma_prep_kernel<2, true, true>), pgrid, dim3(kPrepThreads), 0, stream, dc.pi, dc.s_pi, q, q_dt, n_queries, plan.n_groups, c.key_fix3, qop, nullptr);
    else
      hipLaunchKernelGGL((mfma_prep_kernel<2, false, true>), pgrid, dim3(kPrepThreads), 0, stream, dc.pi, dc.s_pi, q, q_dt, n_queries, plan.n_groups, c.key_fix3, qop, nullptr);
    ScanMfmaArgs a;
    a.qop = reinterpret_cast<const u32x4*>(qop);
    a.records = static_cast<const uint8_t*>(records);
    a.scores = scores;
    a.capacity = capacity;
    a.n_tokens = n_tokens;
    a.rec_bytes = c.rec_bytes;
    a.kbytes = c.kbytes;
    a.norm_off = c.norm_off;
    a.n_queries = n_queries;
    a.n_qtiles = plan.n_groups / 4;
    // 16-byte score stores need 16-byte aligned rows
    a.vec_store = (n_tokens % 4 == 0 && reinterpret_cast<uintptr_t>(scores) % 16 == 0) ? 1 : 0;
    a.inv_sqrt_d = c.inv_sqrt_d;
    a.qjl_coef = c.qjl_coef;
    a.key_fix3 = c.key_fix3;
    for (int i = 0; i < kMaxLevels; ++i) a.key_levels[i] = c.key_levels[i];
    const dim3 grid((unsigned)((n_tokens + kScanBlockTok - 1) / kScanBlockTok),
                    (unsigned)((a.n_qtiles + kScanQT - 1) / kScanQT), (unsigned)(batch * heads));
    ev.before(stream);
    if (c.kb == 3 && qjl) launch_scan_mfma<3, true>(grid, a, stream);
    else if (c.kb == 3) launch_scan_mfma<3, false>(grid, a, stream);
    else if (qjl) launch_scan_mfma<2, true>(grid, a, stream);
    else launch_scan_mfma<2, false>(grid, a, stream);
    ev.after(stream);
    return hipGetLastError();
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* qh = reinterpret_cast<uint16_t*>(ws + plan.ws_q);
  uint16_t* ql = reinterpret_cast<uint16_t*>(ws + plan.ws_ql);
  float* qscale = reinterpret_cast<float*>(ws + plan.ws_qscale);
  const int rows = batch * heads * n_queries;
  const float sfix = std::ldexp(1.0f, (int)std::lround(0.5 * std::log2((double)c.d)));   // ~sqrt(d)
  hipLaunchKernelGGL(scan_prep_f16_kernel, dim3(rows), dim3(kScanPrepThreads), 0, stream, dc.pi, dc.s, c.d, c.m, plan.kp, sfix,
                     q, q_dt, qh, ql, qscale);
  Scan16Args a;
  a.qh = qh;
  a.ql = ql;
  a.qscale = qscale;
  a.records = static_cast<const uint8_t*>(records);
  a.scores = scores;
  a.capacity = capacity;
  a.n_tokens = n_tokens;
  a.d = c.d;
  a.m = c.m;
  a.kp = plan.kp;
  a.kb = c.kb;
  a.kbytes = c.kbytes;
  a.rec_bytes = c.rec_bytes;
  a.norm_off = c.norm_off;
  a.n_queries = n_queries;
  a.inv_sqrt_d = c.inv_sqrt_d;
  a.qjl_coef = c.qjl_coef;
  a.gmax = 0.0f;
  a.sfix = sfix;
  for (int i = 0; i < kMaxLevels; ++i) {
    a.key_levels[i] = c.key_levels[i];
    if (i < (1 << c.kb)) a.gmax = std::max(a.gmax, std::fabs(c.key_levels[i]));
  }
  dim3 grid((unsigned)((n_tokens + kS16Tile - 1) / kS16Tile), (unsigned)((n_queries + kS16Tile - 1) / kS16Tile),
            (unsigned)(batch * heads));
  ev.before(stream);
  a.pcs = dc.polar.cs64;
  a.pb1 = c.pb1;
  a.pbh = c.pbh;
  a.plevels = c.plevels;
  a.l1_bytes = c.l1_bytes;
  if (c.polar)
    hipLaunchKernelGGL(scan_mfma16_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(scan_mfma16_kernel<false>, grid, dim3(256), 0, stream, a);
  ev.after(stream);
  return hipGetLastError();
}

// =========================================================================================
// Measurement support: a streaming read of `bytes` bytes.  Each of ~16 workgroups per CU reads
// one contiguous slice with 16-byte loads, eight in flight per thread, and folds it into one
// word per wave so the loads cannot be dropped.  It gives the bench its own read ceiling.
// =========================================================================================
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* sink) {
  constexpr int U = 8;
  uint32_t x = 0;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = min((size_t)blockIdx.x * per, n16), b1 = min(b0 + per, n16);
  size_t i = b0 + threadIdx.x;
  for (; i + (U - 1) * 256 < b1; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < b1; i += 256) {
    const u32x4 a = src[i];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
#pragma unroll
  for (int msk = 32; msk > 0; msk >>= 1) x ^= __shfl_xor(x, msk);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = x;
}

int stream_read_blocks() { return 16 * num_cus(); }
size_t stream_read_sink_words() { return (size_t)stream_read_blocks() * 4; }

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream,
                              const ProfileEvents& ev) {
  ev.before(stream);
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  ev.after(stream);
  return hipGetLastError();
}

// =========================================================================================
// Hot/cold step (Monarch v3 page, "Wie es funktioniert" and its decode loop): recent tokens
// exact in a per-sequence ring, older ones compressed; a query head reads the cold region only
// when its best hot logit is below a gate; cold tokens that keep a large attention weight for
// several consecutive steps are decompressed back into the ring (page swap); the ring keeps a
// sliding window and compresses its oldest tokens into the cold region.
//   monarch_prep_kernel     append the step's token to the ring, per-head gates
//   (decode)                cold scan (skipped for fully gated KV-head groups) + merge
//   monarch_promote_kernel  sticky counters, dequantize promoted tokens into the ring,
//                           swap-remove them from the cold region
//   monarch_evict_kernel    compress the ring's oldest tokens past the window (float64) and
//                           commit the new state
// =========================================================================================
constexpr int kMonarchMaxHeads = 64;      // query heads per sequence in the promotion kernel
constexpr int kMonarchMaxPromote = 1024;  // promotions per sequence and step

struct MonarchArgs {
  Consts c;
  PolarTables pt;         // polar key codes: angle bounds, float64 cos / sin of the grid levels
  const float* pi;        // [d][d]
  const float* pi_t;      // [d][d] transposed
  const float* s;         // [m][d]
  const float* s_t;       // [d][m] transposed
  const void* q;
  tq_dtype q_dt;
  const void* k_new;
  const void* v_new;
  void* hot_k;
  void* hot_v;
  tq_dtype hot_dt;
  int64_t hot_cap, cold_cap, logit_stride;
  int32_t* hot_start;
  int32_t* hot_len;
  uint8_t* records;
  int32_t* cold_len;
  int32_t* hits;
  int32_t* overflow;
  int32_t* gate;          // [B][Hq]
  const float* logits;    // [B][Hq][logit_stride] cold logits of the step
  const float* lse;       // [B][Hq]
  int32_t* promo_count;   // [B] (workspace)
  int32_t* cold_after;    // [B] (workspace)
  int32_t* gate_out;      // [B][Hq] copy of the gates for the caller (NULL: none)
  uint32_t* promo_w;      // [B][cold_cap] per-token maximum weight over the open heads (float bits)
  int batch, q_heads, kv_heads, G, window, promote_steps;
  float cold_gate, promote_weight, scale;
};

__device__ __forceinline__ void copy_elem(void* dst, const void* src, tq_dtype dt, int64_t di, int64_t si) {
  if (dt == TQ_F32) static_cast<float*>(dst)[di] = static_cast<const float*>(src)[si];
  else static_cast<uint16_t*>(dst)[di] = static_cast<const uint16_t*>(src)[si];
}

// float64 -> float32 rounded to odd (toward zero, low bit set when inexact): a following
// round-to-nearest-even to bf16 / f16 then equals the correctly rounded float64 value.
__device__ __forceinline__ float f64_to_f32_odd(double x) {
  float f = __double2float_rz(x);
  if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f;
}
__device__ __forceinline__ void store_f64(void* base, tq_dtype dt, int64_t off, double x) {
  if (dt == TQ_F32) {
    static_cast<float*>(base)[off] = (float)x;
  } else if (dt == TQ_BF16) {
    const uint32_t u = __float_as_uint(f64_to_f32_odd(x));
    static_cast<uint16_t*>(base)[off] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  } else {
    static_cast<uint16_t*>(base)[off] = __builtin_bit_cast(uint16_t, (_Float16)f64_to_f32_odd(x));
  }
}

// Code j of a packed code field (3-bit: the 32-code group layout; 2/4-bit: bitstream).
__device__ __forceinline__ uint32_t field_code(const uint8_t* field, int j, int bits) {
  if (bits == 3) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(field + 12 * (j >> 5));
    return group3_code(w[0], w[1], w[2], j & 31);
  }
  const int pos = j * bits;
  return (field[pos >> 3] >> (pos & 7)) & ((1u << bits) - 1u);
}

// One record from its codes, sign bits and norms (the layout compress_kernel writes).
__device__ void pack_record(const Consts& c, const uint32_t* ck, const uint32_t* bits, const uint32_t* cv,
                            float rk, float rho, float rv, uint8_t* rec) {
  auto put = [&](uint8_t* field, const uint32_t* codes, int nbits) {
    if (nbits == 3) {
      for (int gi = 0; gi < c.d / 32; ++gi) {
        uint32_t w[3] = {0u, 0u, 0u};
        for (int j = 0; j < 32; ++j) group3_put(w, j, codes[32 * gi + j]);
        uint32_t* dst = reinterpret_cast<uint32_t*>(field + 12 * gi);
        dst[0] = w[0];
        dst[1] = w[1];
        dst[2] = w[2];
      }
    } else {
      ByteWriter w{field, 0, 0};
      for (int i = 0; i < c.d; ++i) w.put(codes[i], nbits);
    }
  };
  if (c.polar) {
    // level-1 angle codes as a pb1-bit stream, then levels 2..L (node order) as a pbh-bit
    // stream zero-padded to the key field's whole words
    ByteWriter w1{rec, 0, 0};
    for (int i = 0; i < c.d / 2; ++i) w1.put(ck[i], c.pb1);
    ByteWriter w2{rec + c.l1_bytes, 0, 0};
    for (int i = c.d / 2; i < c.d - 1; ++i) w2.put(ck[i], c.pbh);
    uint8_t* p = w2.dst;
    if (w2.n > 0) *p++ = (uint8_t)w2.acc;
    while (p < rec + c.kbytes) *p++ = 0;
  } else {
    put(rec, ck, c.kb);
  }
  ByteWriter ws{rec + c.kbytes, 0, 0};
  for (int j = 0; j < c.m; ++j) ws.put(bits[j], 1);
  put(rec + c.kbytes + c.sbytes, cv, c.vb);
  float* nrm = reinterpret_cast<float*>(rec + c.norm_off);
  nrm[0] = rk;
  nrm[1] = rho;
  nrm[2] = rv;
  for (int i = c.norm_off + 12; i < c.rec_bytes; ++i) rec[i] = 0;
}

// Word w of the record pack_record writes, from the same codes, bits and norms: one thread
// per word (b-bit streams with b dividing 32 hold whole codes per word; 3-bit fields are whole
// 32-code groups at the head_dims this serves, 64 and 128).
__device__ uint32_t record_word(const Consts& c, const uint32_t* ck, const uint32_t* bits, const uint32_t* cv,
                                float rk, float rho, float rv, int w) {
  auto stream_word = [](const uint32_t* codes, int n, int nbits, int idx) -> uint32_t {
    const int per = 32 / nbits, first = idx * per;
    uint32_t word = 0;
    for (int i = 0; i < per && first + i < n; ++i) word |= codes[first + i] << (nbits * i);
    return word;
  };
  auto group3_word = [](const uint32_t* codes, int idx) -> uint32_t {
    const int k = idx % 3;
    const uint32_t* cg = codes + 32 * (idx / 3);
    uint32_t word = 0;
    for (int j = 8 * k; j < 8 * k + 8; ++j) word |= cg[j] << (8 * (j & 3) + 3 * ((j >> 2) & 1));
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t t6 = cg[24 + kk] | (cg[28 + kk] << 3);     // codes 24 + kk and 28 + kk
      word |= ((t6 >> (2 * k)) & 3u) << (8 * kk + 6);
    }
    return word;
  };
  const int off = 4 * w;
  if (off < c.kbytes) {
    if (c.polar) {
      const int l1w = c.l1_bytes / 4;
      return w < l1w ? stream_word(ck, c.d / 2, c.pb1, w) : stream_word(ck + c.d / 2, c.d / 2 - 1, c.pbh, w - l1w);
    }
    return c.kb == 3 ? group3_word(ck, w) : stream_word(ck, c.d, c.kb, w);
  }
  if (off < c.kbytes + c.sbytes) return stream_word(bits, c.m, 1, w - c.kbytes / 4);
  if (off < c.kbytes + c.sbytes + c.vbytes) {
    const int vw = w - (c.kbytes + c.sbytes) / 4;
    return c.vb == 3 ? group3_word(cv, vw) : stream_word(cv, c.d, c.vb, vw);
  }
  if (off == c.norm_off) return __float_as_uint(rk);
  if (off == c.norm_off + 4) return __float_as_uint(rho);
  if (off == c.norm_off + 8) return __float_as_uint(rv);
  return 0u;
}

template <int D>
__global__ __launch_bounds__(1024) void monarch_prep_kernel(MonarchArgs M) {
  // lanes split a token's coordinates 8 at a time (LPK lanes per token), as the merge does
  constexpr int LPK = D / 8, TPI = 1024 / LPK;
  __shared__ float qv[16][D];
  __shared__ float red[16][16];
  const int hkv = blockIdx.x, b = blockIdx.y, G = M.G;
  const int64_t unit = (int64_t)b * M.kv_heads + hkv;
  if (M.promo_w && hkv == 0) {    // cleared before the step's merge folds the weights in
    const int nc = (int)min((int64_t)M.cold_len[b], M.cold_cap);
    for (int t = threadIdx.x; t < nc; t += blockDim.x) M.promo_w[(int64_t)b * M.cold_cap + t] = 0u;
  }
  const int n = M.hot_len[b];
  const int64_t st = M.hot_start[b];
  int64_t slot = st + n;
  if (slot >= M.hot_cap) slot -= M.hot_cap;
  for (int i = threadIdx.x; i < D; i += blockDim.x) {
    copy_elem(M.hot_k, M.k_new, M.hot_dt, (unit * M.hot_cap + slot) * D + i, unit * D + i);
    copy_elem(M.hot_v, M.v_new, M.hot_dt, (unit * M.hot_cap + slot) * D + i, unit * D + i);
  }
  const int64_t qrow0 = (int64_t)b * M.q_heads + (int64_t)hkv * G;
  if (M.cold_gate == INFINITY) {      // no gate: every head reads the cold tokens
    if (threadIdx.x < G) M.gate[qrow0 + threadIdx.x] = 1;
    return;
  }
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) qv[e / D][e % D] = load_elem(M.q, M.q_dt, qrow0 * D + e);
  __syncthreads();
  // best hot logit per head over the ring's tokens and the step's token (read from k_new); the
  // next round's keys are loaded while this round's are used
  const int sub = threadIdx.x % LPK, tok = threadIdx.x / LPK;
  float mx[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) mx[j] = kNegInf;
  auto load_key = [&](int t0, float (&kv)[8]) {
    const int t = min(t0 + tok, n);
    int64_t rs = st + t;
    if (rs >= M.hot_cap) rs -= M.hot_cap;
    load8(t < n ? M.hot_k : M.k_new, M.hot_dt, (t < n ? (unit * M.hot_cap + rs) * D : unit * D) + 8 * sub, kv);
  };
  float kn[8];
  load_key(0, kn);
  for (int t0 = 0; t0 <= n; t0 += TPI) {
    float kv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kv[i] = kn[i];
    if (t0 + TPI <= n) load_key(t0 + TPI, kn);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= G) break;
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) dot = fmaf(qv[j][8 * sub + i], kv[i], dot);
#pragma unroll
      for (int msk = 1; msk < LPK; msk <<= 1) dot += __shfl_xor(dot, msk);
      mx[j] = fmaxf(mx[j], M.scale * dot);    // tokens past n repeat token n: the max is unchanged
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j >= G) break;
    float v = mx[j];
#pragma unroll
    for (int msk = 32; msk > 0; msk >>= 1) v = fmaxf(v, __shfl_xor(v, msk));
    if (lane == 0) red[wave][j] = v;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float v = red[0][threadIdx.x];
    for (int w2 = 1; w2 < 16; ++w2) v = fmaxf(v, red[w2][threadIdx.x]);
    M.gate[qrow0 + threadIdx.x] = v < M.cold_gate ? 1 : 0;
  }
}

template <int D>
__global__ __launch_bounds__(1024) void monarch_promote_kernel(MonarchArgs M) {
  __shared__ int s_gate[kMonarchMaxHeads];
  __shared__ int plist[kMonarchMaxPromote];
  __shared__ int moves[kMonarchMaxPromote][2];
  __shared__ int wsum[16];
  __shared__ int s_np;
  __shared__ double lev[2][D];
  const int b = blockIdx.x, Hq = M.q_heads;
  const int n_cold = M.cold_len[b];
  for (int h = threadIdx.x; h < Hq; h += blockDim.x) {
    s_gate[h] = M.gate[(int64_t)b * Hq + h];
    if (M.gate_out) M.gate_out[(int64_t)b * Hq + h] = s_gate[h];
  }
  if (threadIdx.x == 0) s_np = 0;
  __syncthreads();
  int32_t* hits = M.hits + (int64_t)b * M.cold_cap;
  if (M.promote_steps > 0) {
    // two consecutive tokens per thread (2,048 per pass).  A token's weight, the largest
    // exp(logit - lse) over the open heads, was folded into promo_w by the heads' merges (0 when
    // no head is open)
    const uint32_t* pw = M.promo_w + (int64_t)b * M.cold_cap;
    for (int t0 = 0; t0 < n_cold; t0 += 2 * blockDim.x) {
      const int ta = t0 + 2 * threadIdx.x;
      bool prom[2] = {false, false};
      int hv[2];
      float w[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        hv[k] = hits[min(ta + k, max(n_cold - 1, 0))];
        w[k] = __uint_as_float(pw[min(ta + k, max(n_cold - 1, 0))]);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (ta + k < n_cold) {
          const int hc = w[k] >= M.promote_weight ? hv[k] + 1 : 0;
          prom[k] = hc >= M.promote_steps;
          hits[ta + k] = prom[k] ? 0 : hc;
        }
      }
      int tot;
      const int pos = block_exclusive_sum<1024>((prom[0] ? 1 : 0) + (prom[1] ? 1 : 0), wsum, &tot);
      if (prom[0] && s_np + pos < kMonarchMaxPromote) plist[s_np + pos] = ta;
      if (prom[1] && s_np + pos + (prom[0] ? 1 : 0) < kMonarchMaxPromote) plist[s_np + pos + (prom[0] ? 1 : 0)] = ta + 1;
      __syncthreads();
      if (threadIdx.x == 0) s_np = min(s_np + tot, kMonarchMaxPromote);
      __syncthreads();
    }
  }
  const int P = s_np;
  // dequantize the promoted tokens (ascending cold index) into the ring after the step's token:
  // k = Pi^T ((r_k / sqrt(d)) gamma_k[c]), v = Pi^T ((r_v / sqrt(d)) gamma_v[c_v]), float64
  const Consts& c = M.c;
  const int64_t st = M.hot_start[b], n_hot = (int64_t)M.hot_len[b] + 1;
  for (int pi = 0; pi < P; ++pi) {
    for (int h = 0; h < M.kv_heads; ++h) {
      const int64_t unit = (int64_t)b * M.kv_heads + h;
      const uint8_t* rec = M.records + (unit * M.cold_cap + plist[pi]) * c.rec_bytes;
      const float* nrm = reinterpret_cast<const float*>(rec + c.norm_off);
      for (int i = threadIdx.x; i < 2 * D; i += blockDim.x) {
        if (i < D && c.polar) {
          // r_k u_i, u_i the product of the cos / sin factors on coordinate i's path from the
          // root (root first, as the inverse transform multiplies)
          double u = 1.0;
          for (int l = c.plevels; l >= 1; --l) {
            const int node = i >> l, side = (i >> (l - 1)) & 1;
            const int bits = l == 1 ? c.pb1 : c.pbh;
            const int idx = l == 1 ? node : (D - (D >> (l - 1)) + node) - D / 2;
            const uint8_t* fld = l == 1 ? rec : rec + c.l1_bytes;
            const uint32_t code = (fld[(idx * bits) >> 3] >> ((idx * bits) & 7)) & ((1u << bits) - 1u);
            u = mul64(u, M.pt.cs64[2 * ((l - 1) * 16 + code) + side]);
          }
          lev[0][i] = mul64((double)nrm[0], u);
        } else if (i < D) {
          lev[0][i] = ((double)nrm[0] / c.sqrt_d) * (double)c.key_levels[field_code(rec, i, c.kb)];
        } else {
          lev[1][i - D] = ((double)nrm[2] / c.sqrt_d) *
                          (double)c.val_levels[field_code(rec + c.kbytes + c.sbytes, i - D, c.vb)];
        }
      }
      __syncthreads();
      int64_t slot = st + n_hot + pi;
      slot %= M.hot_cap;
      for (int i = threadIdx.x; i < 2 * D; i += blockDim.x) {
        const int which = i / D, o = i % D;
        // row o of Pi^T read as column o of Pi (contiguous across the lanes' o)
        double acc = 0.0;
        for (int j0 = 0; j0 < D; j0 += 32) {      // 32 loads in flight
          float pv[32];
#pragma unroll
          for (int u = 0; u < 32; ++u) pv[u] = M.pi[(j0 + u) * D + o];
#pragma unroll
          for (int u = 0; u < 32; ++u) acc = fma((double)pv[u], lev[which][j0 + u], acc);
        }
        store_f64(which ? M.hot_v : M.hot_k, M.hot_dt, (unit * M.hot_cap + slot) * D + o, acc);
      }
      __syncthreads();
    }
  }
  // swap-remove in descending index order: the current last cold token fills each hole
  if (threadIdx.x == 0) {
    int nc = n_cold;
    for (int i = P - 1; i >= 0; --i) {
      const int p = plist[i], last = nc - 1;
      moves[i][0] = last;
      moves[i][1] = p;
      --nc;
    }
  }
  __syncthreads();
  // each thread owns the same 16-byte pieces of a token's records in every move (program order
  // keeps the chain of moves consistent without cross-thread synchronisation)
  const int pieces = M.kv_heads * (c.rec_bytes / 16);
  for (int i = P - 1; i >= 0; --i) {
    const int src = moves[i][0], dst = moves[i][1];
    if (src == dst) continue;
    for (int e = threadIdx.x; e < pieces; e += blockDim.x) {
      const int h = e / (c.rec_bytes / 16), pc = e % (c.rec_bytes / 16);
      const int64_t unit = (int64_t)b * M.kv_heads + h;
      const u32x4* s4 = reinterpret_cast<const u32x4*>(M.records + (unit * M.cold_cap + src) * c.rec_bytes) + pc;
      u32x4* d4 = reinterpret_cast<u32x4*>(M.records + (unit * M.cold_cap + dst) * c.rec_bytes) + pc;
      *d4 = *s4;
    }
    if (threadIdx.x == 0) hits[dst] = hits[src];
  }
  if (threadIdx.x == 0) {
    M.promo_count[b] = P;
    M.cold_after[b] = n_cold - P;
  }
}

// Eviction: every KV head of an evicted token at once.  Threads split (head, K/V, coordinate)
// work in each phase; float64 throughout, as compress_kernel and the oracle.
constexpr int kMonarchMaxKvHeads = 16;

// sketch-bit slots per head in the eviction's LDS, even so that what follows stays 8-byte aligned
__host__ __device__ constexpr int c_m_words(int m) { return (m + 1) / 2 * 2; }

template <int D>
__global__ __launch_bounds__(512) void monarch_evict_kernel(MonarchArgs M) {
  constexpr int HM = kMonarchMaxKvHeads;
  extern __shared__ __attribute__((aligned(16))) double ev_lds[];
  double* vin = ev_lds;                         // [H][2][D] inputs (K, V)
  double* xr = vin + HM * 2 * D;                // [H][2][D] rotated
  double* er = xr + HM * 2 * D;                 // [H][D] key residual
  uint32_t* codes = reinterpret_cast<uint32_t*>(er + HM * D);   // [H][2][D]
  uint32_t* bits = codes + HM * 2 * D;          // [H][m]
  double* pr = reinterpret_cast<double*>(bits + HM * c_m_words(M.c.m));   // [H][D] polar radii / scales
  __shared__ double nrm[HM][3];                 // r_k, r_v (float64), rho
  const int b = blockIdx.x, H = M.kv_heads;
  const Consts& c = M.c;
  const int64_t st = M.hot_start[b];
  const int n_hot = M.hot_len[b] + 1 + M.promo_count[b];
  const int e = max(0, n_hot - M.window);
  const int c0 = M.cold_after[b];
  const int es = (int)min((int64_t)e, M.cold_cap - c0);
  for (int i = 0; i < es; ++i) {
    int64_t rs = st + i;
    rs %= M.hot_cap;
    // inputs
    for (int t = threadIdx.x; t < H * 2 * D; t += blockDim.x) {
      const int h = t / (2 * D), w = (t / D) & 1, j = t % D;
      const int64_t unit = (int64_t)b * H + h;
      vin[t] = (double)load_elem(w ? M.hot_v : M.hot_k, M.hot_dt, (unit * M.hot_cap + rs) * D + j);
    }
    __syncthreads();
    // norms r_k, r_v
    for (int t = threadIdx.x; t < H * 2; t += blockDim.x) {
      double s = 0.0;
      for (int j = 0; j < D; ++j) s = fma(vin[t * D + j], vin[t * D + j], s);
      nrm[t >> 1][t & 1] = sqrt(s);
    }
    __syncthreads();
    // rotation and codes: z = (Pi x) sqrt(d) / r rounded to float32
    for (int t = threadIdx.x; t < H * 2 * D; t += blockDim.x) {
      const int h = t / (2 * D), w = (t / D) & 1, o = t % D;
      const double* xv = vin + (h * 2 + w) * D;
      // row o of Pi read as column o of Pi^T: for each j the lanes (consecutive o) read one
      // contiguous run; four partial sums keep the dependency chains short
      double a4[4] = {0.0, 0.0, 0.0, 0.0};
      for (int j0 = 0; j0 < D; j0 += 64) {        // 64 loads in flight
        float pv[64];
#pragma unroll
        for (int u = 0; u < 64; ++u) pv[u] = M.pi_t[(j0 + u) * D + o];
#pragma unroll
        for (int u = 0; u < 64; ++u) a4[u & 3] = fma((double)pv[u], xv[j0 + u], a4[u & 3]);
      }
      const double acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
      xr[t] = acc;
      const double r = nrm[h][w];
      const double scale = r > 0.0 ? c.sqrt_d / r : 0.0;
      if (w || !c.polar) codes[t] = quantize_code((float)(acc * scale), w ? c.val_bounds : c.key_bounds);
    }
    __syncthreads();
    if (c.polar) {
      // polar key codes (TurboQuant page, "PolarQuant"), level by level with one thread per
      // node: level l node i has its code and radius at index D - (D >> (l - 1)) + i
      const int nb1 = (1 << c.pb1) - 1, nbh = (1 << c.pbh) - 1;
      for (int l = 1; l <= c.plevels; ++l) {
        const int cnt = D >> l, off = D - (D >> (l - 1)), coff = l == 1 ? 0 : D - (D >> (l - 2));
        for (int t = threadIdx.x; t < H * cnt; t += blockDim.x) {
          const int h = t / cnt, i = t % cnt;
          const double a = l == 1 ? xr[h * 2 * D + 2 * i] : pr[h * D + coff + 2 * i];
          const double bv = l == 1 ? xr[h * 2 * D + 2 * i + 1] : pr[h * D + coff + 2 * i + 1];
          codes[h * 2 * D + off + i] = polar_code(polar_angle(a, bv), M.pt.bounds + (l - 1) * 16, l == 1 ? nb1 : nbh);
          pr[h * D + off + i] = sqrt(add64(mul64(a, a), mul64(bv, bv)));
        }
        __syncthreads();
      }
      // the unit vector of the grid angles, top-down: a node's scale times the cos / sin of its
      // angle is its children's (root scale 1, the multiplication order of the inverse transform)
      for (int h = threadIdx.x; h < H; h += blockDim.x) pr[h * D + D - 2] = 1.0;
      __syncthreads();
      for (int l = c.plevels; l >= 2; --l) {
        const int cnt = D >> l, off = D - (D >> (l - 1)), coff = D - (D >> (l - 2));
        for (int t = threadIdx.x; t < H * cnt; t += blockDim.x) {
          const int h = t / cnt, i = t % cnt;
          const double sc = pr[h * D + off + i];
          const double* cs = M.pt.cs64 + 2 * ((l - 1) * 16 + codes[h * 2 * D + off + i]);
          pr[h * D + coff + 2 * i] = mul64(sc, cs[0]);
          pr[h * D + coff + 2 * i + 1] = mul64(sc, cs[1]);
        }
        __syncthreads();
      }
      // key residual e = y - r_k u with r_k stored as float32
      for (int t = threadIdx.x; t < H * D; t += blockDim.x) {
        const int h = t / D, j = t % D;
        const double* cs = M.pt.cs64 + 2 * codes[h * 2 * D + (j >> 1)];
        const double u = mul64(pr[h * D + (j >> 1)], cs[j & 1]);
        er[t] = sub64(xr[h * 2 * D + j], mul64((double)(float)nrm[h][0], u));
      }
      __syncthreads();
    } else {
      // key residual e = x - (r_k / sqrt(d)) gamma[c] with r_k stored as float32
      for (int t = threadIdx.x; t < H * D; t += blockDim.x) {
        const int h = t / D, j = t % D;
        const double rk = (double)(float)nrm[h][0];
        er[t] = xr[h * 2 * D + j] - (rk / c.sqrt_d) * (double)c.key_levels[codes[h * 2 * D + j]];
      }
      __syncthreads();
    }
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
      double s = 0.0;
      for (int j = 0; j < D; ++j) s = fma(er[h * D + j], er[h * D + j], s);
      nrm[h][2] = sqrt(s);
    }
    // QJL signs of S e
    for (int t = threadIdx.x; t < H * c.m; t += blockDim.x) {
      const int h = t / c.m, j = t % c.m;
      double a4[4] = {0.0, 0.0, 0.0, 0.0};
      for (int k0 = 0; k0 < D; k0 += 64) {        // row j of S as column j of S^T, 64 loads in flight
        float sv[64];
#pragma unroll
        for (int u = 0; u < 64; ++u) sv[u] = M.s_t[(k0 + u) * c.m + j];
#pragma unroll
        for (int u = 0; u < 64; ++u) a4[u & 3] = fma((double)sv[u], er[h * D + k0 + u], a4[u & 3]);
      }
      const double acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
      bits[t] = (float)acc >= 0.0f ? 1u : 0u;
    }
    __syncthreads();
    // the records, one thread per (head, 32-bit word)
    const int nw = c.rec_bytes / 4;
    for (int t = threadIdx.x; t < H * nw; t += blockDim.x) {
      const int h = t / nw, w = t % nw;
      const int64_t unit = (int64_t)b * H + h;
      reinterpret_cast<uint32_t*>(M.records + (unit * M.cold_cap + c0 + i) * c.rec_bytes)[w] =
          record_word(c, codes + h * 2 * D, bits + h * c.m, codes + h * 2 * D + D, (float)nrm[h][0],
                      (float)nrm[h][2], (float)nrm[h][1], w);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int32_t* hits = M.hits + (int64_t)b * M.cold_cap;
    for (int i = 0; i < es; ++i) hits[c0 + i] = 0;
    M.hot_start[b] = (int32_t)((st + e) % M.hot_cap);
    M.hot_len[b] = n_hot - e;
    M.cold_len[b] = c0 + es;
    if (es < e) M.overflow[b] = 1;
  }
}

template <int D>
size_t monarch_evict_lds(int m) {
  return (size_t)kMonarchMaxKvHeads * (2 * D * 8 * 2 + D * 8 + 2 * D * 4 + (size_t)c_m_words(m) * 4 + D * 8);
}

MonarchPlan plan_monarch(const Consts& c, int batch, int q_heads, int kv_heads, int64_t hot_cap,
                         int64_t cold_cap, bool* ok) {
  MonarchPlan p;
  *ok = plan_decode(c, batch, q_heads, kv_heads, cold_cap, &p.decode);
  const size_t rows = (size_t)std::max(batch, 1) * q_heads;
  p.logit_stride = cold_cap + hot_cap;
  p.ws_decode = 0;
  p.ws_gate = align256(p.decode.ws_total);
  p.ws_lse = p.ws_gate + align256(rows * 4);
  p.ws_logits = p.ws_lse + align256(rows * 4);
  p.ws_counts = p.ws_logits + align256(rows * (size_t)p.logit_stride * 4);
  p.ws_promo = p.ws_counts + align256((size_t)std::max(batch, 1) * 8);
  p.ws_total = p.ws_promo + align256((size_t)std::max(batch, 1) * (size_t)cold_cap * 4);
  return p;
}

hipError_t launch_monarch_step(const Consts& c, const DevConsts& dc, const MonarchPlan& plan,
                               const MonarchStep& s, void* workspace, hipStream_t stream,
                               const ProfileEvents& ev) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  MonarchArgs M;
  M.c = c;
  M.pi = dc.pi;
  M.pi_t = dc.pi_t;
  M.s = dc.s;
  M.s_t = dc.s_t;
  M.q = s.q;
  M.q_dt = s.q_dt;
  M.k_new = s.k_new;
  M.v_new = s.v_new;
  M.hot_k = s.hot_k;
  M.hot_v = s.hot_v;
  M.hot_dt = s.hot_dt;
  M.hot_cap = s.hot_cap;
  M.cold_cap = s.cold_cap;
  M.logit_stride = plan.logit_stride;
  M.hot_start = s.hot_start;
  M.hot_len = s.hot_len;
  M.records = static_cast<uint8_t*>(s.records);
  M.cold_len = s.cold_len;
  M.hits = s.hits;
  M.overflow = s.overflow;
  M.gate_out = s.gate_out;
  M.gate = reinterpret_cast<int32_t*>(ws + plan.ws_gate);
  float* lse = s.lse ? s.lse : reinterpret_cast<float*>(ws + plan.ws_lse);
  float* logits = reinterpret_cast<float*>(ws + plan.ws_logits);
  M.logits = logits;
  M.lse = lse;
  M.promo_count = reinterpret_cast<int32_t*>(ws + plan.ws_counts);
  M.promo_w = s.promote_steps > 0 ? reinterpret_cast<uint32_t*>(ws + plan.ws_promo) : nullptr;
  M.cold_after = M.promo_count + std::max(s.batch, 1);
  M.batch = s.batch;
  M.q_heads = s.q_heads;
  M.kv_heads = s.kv_heads;
  M.G = s.q_heads / s.kv_heads;
  M.window = s.window;
  M.promote_steps = s.promote_steps;
  M.cold_gate = s.cold_gate;
  M.promote_weight = s.promote_weight;
  M.scale = s.scale > 0.0f ? s.scale : c.inv_sqrt_d;
  M.pt = dc.polar;
  const dim3 g1(s.kv_heads, s.batch);
  if (c.d == 128) hipLaunchKernelGGL(monarch_prep_kernel<128>, g1, dim3(1024), 0, stream, M);
  else hipLaunchKernelGGL(monarch_prep_kernel<64>, g1, dim3(1024), 0, stream, M);
  DecodeHooks hk{M.gate, s.hot_start, 1, M.promo_w};
  hipError_t e = launch_decode(c, dc, plan.decode, s.q, s.q_dt, s.batch, s.q_heads, s.kv_heads, s.records,
                               s.cold_cap, s.cold_len, s.hot_k, s.hot_v, s.hot_dt, s.hot_len, s.hot_cap,
                               nullptr, 0, M.scale, s.out, lse, logits, ws + plan.ws_decode, stream, ev, &hk);
  if (e != hipSuccess) return e;
  if (c.d == 128) {
    hipLaunchKernelGGL(monarch_promote_kernel<128>, dim3(s.batch), dim3(1024), 0, stream, M);
    const size_t lds = monarch_evict_lds<128>(c.m);
    allow_lds(monarch_evict_kernel<128>, lds);
    hipLaunchKernelGGL(monarch_evict_kernel<128>, dim3(s.batch), dim3(512), lds, stream, M);
  } else {
    hipLaunchKernelGGL(monarch_promote_kernel<64>, dim3(s.batch), dim3(1024), 0, stream, M);
    const size_t lds = monarch_evict_lds<64>(c.m);
    allow_lds(monarch_evict_kernel<64>, lds);
    hipLaunchKernelGGL(monarch_evict_kernel<64>, dim3(s.batch), dim3(512), lds, stream, M);
  }
  return hipGetLastError();
}


// -----------------------------------------------------------------------------------------
// Fixed scratch of the allocation-free decode.  In host code `scratch` names a host-side
// stand-in, not device memory: kernels and copies only ever get the device address that
// hipGetSymbolAddress returns (one per device, looked up once with that device current).
// -----------------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kScratchMaxDevices];

hipError_t scratch_setup() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev]) return hipSuccess;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256 != 0) return hipErrorInvalidSymbol;
  g_scratch_ptr[dev] = ptr;
  return hipSuccess;
}

void* scratch_address(int device) {
  if (device < 0 || device >= kScratchMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

}  // namespace tq
