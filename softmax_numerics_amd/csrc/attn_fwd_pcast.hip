// FP8 "P-cast" attention for MI355X (gfx950 / CDNA4): the forward, and around it.
//
// What is computed (FlashAttention blog, "L'algoritmo Flash Attention" and
// "La ricorrenza softmax online"; P-cast summaries, sections 1-2): for every
// query row, key blocks of 64 are visited forward or in reverse; the running
// max m' includes the current block; P = exp(s - m') is summed un-cast into l;
// P*S is rounded to E4M3 and multiplied with E4M3(V) on the FP8 matrix cores;
// the accumulator is rescaled by exp(m - m') when the max grows and divided by
// S*l at the end.  S = 0 (no cast) runs a separate kernel with P and V in bf16.
//
// Mapping to CDNA4:
// * One workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//   owns 32 rows.  Logits are formed transposed, S^T = K Q^T, on
//   v_mfma_f32_32x32x16_bf16, so each lane's accumulator column is one query
//   row: lane l holds row l%32 and 32 of the block's 64 keys, lane l^32 the
//   other 32.  Row max / row sum need one cross-lane exchange per block.
// * The output is accumulated transposed too, O^T += V^T P^T, on
//   v_mfma_f32_32x32x64_f8f6f4 (K = 64 = one key block per instruction), so
//   the per-row rescale factor is a per-lane scalar.
// * The P codes never leave registers: the order in which a lane holds its 32
//   keys is taken as the MFMA's k order, and V is copied once per call (by
//   pcast_prep_v) into E4M3 in the same key order, transposed to [d][key], so
//   both operands agree without any shuffle.
// * K and V tiles are staged through LDS by direct global->LDS loads, double
//   buffered, each buffer its own LDS object.  The FP8 kernel is software-
//   pipelined by one block: step j holds block j-1's P.V, block j's softmax
//   and block j+1's logits, interleaved MFMA by MFMA.
// * Exactness of the scale: for S = 2^k the product P*S is formed inside the
//   conversion (v_cvt_scalef32_pk_fp8_f32 with scale 2^-k), which is exact;
//   1/(S*l) is exact up to the final reciprocal.  Other S use an fp32 multiply
//   (not exact, as the P-cast summary notes for 448), and S > 448 clamps first
//   because the conversion does not saturate by itself.
//
// Around the forward, in this file:
// * FP8 logits: a template flag of the FP8 kernel rounds Q to E4M3 per row as
//   it loads it and reads K as E4M3 codes with one scale per key block
//   (pcast_prep_kv8 writes them, with the V copy); the logits then run on the
//   FP8 matrix cores too.
// * Row diagnostics: a counter level of the FP8 kernel that also accumulates the
//   non-sink and the zeroed non-sink mass of each row and writes its lse.
// * Split-KV decode: pcast_decode_split (one wave per key range, GQA rows packed
//   into the MFMA columns) and pcast_decode_merge.
// * Backward by recomputation from lse: pcast_bwd_rowdot, pcast_attn_bwd_dq (a
//   lane per query row) and pcast_attn_bwd_dkv (a lane per key); the transposed
//   operands come from ds_read_b64_tr_b16 reads of the row-major tiles.
// * The host side: argument checks, workspace layouts and the C entry points.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <utility>

#include "pcast_attn.h"

// Scratch memory of attn_fwd_pcast_noalloc: the V operand copy of one call.  Each
// device the library runs on holds its own copy until the process ends; host code
// reaches it only through the address hipGetSymbolAddress returns for the current
// device (the name itself is a host-side stand-in, not a device address).
static __device__ __align__(256) uint8_t scratch[PCAST_NOALLOC_SCRATCH_BYTES];

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(2))) short s16x2_t;

constexpr int kKvBlock = PCAST_KV_BLOCK;  // keys per block
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBlockRows = kWaves * kRowsPerWave;  // 128 query rows per workgroup
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Key (within a 64-key block) held by lane group g (= lane / 32) in operand
// slot b (0..31).  It is the order of the S^T accumulator: register r of
// accumulator kb holds key kb*32 + (r/4)*8 + g*4 + r%4, and slot b = kb*16 + r.
__host__ __device__ constexpr int slot_key(int g, int b) {
  return (b >> 4) * 32 + ((b & 15) >> 2) * 8 + g * 4 + (b & 3);
}

template <int D>
struct Geometry {
  static constexpr int kQSteps = D / 16;       // bf16 MFMA k-steps over d
  static constexpr int kDTiles = D / 32;       // 32-column output tiles
};

// An LDS tile of rows of kRowBytes, stored without padding: the 16-byte chunk c of
// row r sits at chunk position c ^ key(r), key(r) = (r / rows per 256 bytes) % chunks
// per row.  The 16 lanes of one ds_read_b128 phase that read the same logical chunk
// of 16 consecutive rows then cover all 64 banks.
template <int kRowBytes>
struct Swizzle {
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kRowsPerWindow = kRowBytes >= 256 ? 1 : 256 / kRowBytes;
  __device__ static int key(int row) { return (row / kRowsPerWindow) % kChunks; }
};

// The backward's row-major tiles use another key: 16 consecutive rows take distinct
// keys (row reads of one 16-byte chunk per lane stay conflict-free), and 4
// consecutive rows fall in 4 different 64-byte windows of the 256-byte bank row
// (the transposing reads take 4 rows x 64 bytes per half wave).
template <int kRowBytes>
struct SwizzleT {
  static_assert(kRowBytes == 256 || kRowBytes == 128, "d = 128 or 64");
  static constexpr int kChunks = kRowBytes / 16;
  __device__ static int key(int row) {
    if constexpr (kChunks == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
};

// ---------------------------------------------------------------------------
// Pre-pass: V (bf16, [B][Hkv][N][D]) -> operand copy [B][Hkv][ceil(N/64)][D][64]
// in slot order, E4M3 (RNE, saturating) or bf16.  Keys past N in a partial last
// block are written as zeros (their probabilities are 0).
// ---------------------------------------------------------------------------
template <int D, bool kFp8>
__device__ inline void prep_v_block(const uint16_t* __restrict__ V, void* __restrict__ vop, int64_t blk, int N,
                                    int n_tiles) {
  __shared__ uint16_t tile[kKvBlock][D + 2];
  const int tid = threadIdx.x;
  const int64_t bh = blk / n_tiles;
  const int t = (int)(blk % n_tiles);
  const int rows = min(kKvBlock, N - t * kKvBlock);  // keys of this block inside the sequence
  const uint16_t* src = V + (bh * N + (int64_t)t * kKvBlock) * D;
  for (int c = tid; c < kKvBlock * D / 8; c += 256) {
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    const i32x4_t v = row < rows ? *reinterpret_cast<const i32x4_t*>(src + row * D + col) : i32x4_t{0, 0, 0, 0};
    const uint32_t w[4] = {(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[row][col + 2 * e] = (uint16_t)(w[e] & 0xFFFFu);
      tile[row][col + 2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
  if constexpr (kFp8) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(vop) + blk * kKvBlock * D);
    for (int w = tid; w < D * 16; w += 256) {
      const int col = w / 16, quad = w % 16;          // 4 slots per word
      const int g = quad / 8, b = (quad % 8) * 4;
      const int k0 = slot_key(g, b);                  // slots b..b+3 are keys k0..k0+3
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = (uint32_t)tile[k0 + e][col] << 16;
        f[e] = fminf(fmaxf(__builtin_bit_cast(float, u), -448.0f), 448.0f);
      }
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], word, true);
      dst[col * 16 + quad] = (uint32_t)word;
    }
  } else {
    uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(vop) + blk * kKvBlock * D);
    for (int w = tid; w < D * 32; w += 256) {
      const int col = w / 32, pair = w % 32;          // 2 slots per word
      const int g = pair / 16, b = (pair % 16) * 2;
      const int k0 = slot_key(g, b);
      dst[col * 32 + pair] = (uint32_t)tile[k0][col] | ((uint32_t)tile[k0 + 1][col] << 16);
    }
  }
}

template <int D, bool kFp8>
__global__ __launch_bounds__(256) void pcast_prep_v(const uint16_t* __restrict__ V,
                                                     void* __restrict__ vop, int N, int n_tiles) {
  prep_v_block<D, kFp8>(V, vop, blockIdx.x, N, n_tiles);  // one (b, hkv, key block) per workgroup
}

// ---------------------------------------------------------------------------
// FP8 logits (an extension of the P-cast path): Q and K rounded to E4M3 with a
// power-of-two scale per block -- per query row for Q, per 64-key block for K.
// The scale of a block is the smallest 2^e with max|x| <= 448 * 2^e, so
// x * 2^-e is exact and never exceeds 448, and the E4M3 conversion (RNE) never
// saturates.
// ---------------------------------------------------------------------------
__device__ inline int scale_exp(uint32_t amax_bits) {  // amax as fp32 bits
  const float a = __builtin_bit_cast(float, amax_bits);
  if (a == 0.0f) return 0;
  int E;
  const float m = frexpf(a, &E);  // a = m * 2^E, m in [0.5, 1); 448 = 0.875 * 2^9
  return m <= 0.875f ? E - 9 : E - 8;
}

// max |x| over the 8 bf16 values in w, as fp32 bits (bf16 bits << 16 order as floats)
__device__ inline uint32_t absmax8(const i32x4_t w) {
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) m = max(m, max((uint32_t)w[e] & 0x7FFFu, ((uint32_t)w[e] >> 16) & 0x7FFFu));
  return m << 16;
}

// E4M3 codes of x * 2^-e for the 8 bf16 values in w, in order, 4 per word
__device__ inline void codes8(const i32x4_t w, int e, int& lo, int& hi) {
  float f[8];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f[2 * t] = ldexpf(__builtin_bit_cast(float, (uint32_t)w[t] << 16), -e);
    f[2 * t + 1] = ldexpf(__builtin_bit_cast(float, (uint32_t)w[t] & 0xFFFF0000u), -e);
  }
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
}

// One key block of K per workgroup: the block's exponent e and the codes of
// K * 2^-e, [B][Hkv][ceil(N/64)*64][D] bytes (the rows past N of a partial last block
// are zeros, which leave its max unchanged), plus the V operand copy of the same block.
template <int D>
__global__ __launch_bounds__(256) void pcast_prep_kv8(const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V,
                                                      uint8_t* __restrict__ vop, uint8_t* __restrict__ k8,
                                                      int* __restrict__ kexp, int N, int n_tiles) {
  constexpr int kChunks = kKvBlock * D / 8 / 256;  // 16-byte chunks per thread
  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;  // flat (b, hkv, key block)
  const int64_t bh = blk / n_tiles;
  const int t = (int)(blk % n_tiles);
  const int rows = min(kKvBlock, N - t * kKvBlock);  // keys of this block inside the sequence
  const uint16_t* src = K + (bh * N + (int64_t)t * kKvBlock) * D;
  i32x4_t w[kChunks];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int e0 = (i * 256 + tid) * 8;  // first element of the chunk in the block
    w[i] = e0 / D < rows ? *reinterpret_cast<const i32x4_t*>(src + e0) : i32x4_t{0, 0, 0, 0};
    m = max(m, absmax8(w[i]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t part[4];
  if (tid % 64 == 0) part[tid / 64] = m;
  __syncthreads();
  const int e = scale_exp(max(max(part[0], part[1]), max(part[2], part[3])));
  uint8_t* dst = k8 + blk * kKvBlock * D;
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    int lo, hi;
    codes8(w[i], e, lo, hi);
    *reinterpret_cast<int2*>(dst + (i * 256 + tid) * 8) = make_int2(lo, hi);
  }
  if (tid == 0) kexp[blk] = e;
  prep_v_block<D, true>(V, vop, blk, N, n_tiles);
}

// Rotated FP8 logits: x -> x diag(sigma) H (H the Sylvester matrix of +-1, sigma the
// caller's signs), in fp64, where the rotation of bf16 inputs is exact; then the
// E4M3 codes of x * 2^-e with one scale per row (kPerRow, for Q) or per 64-row block
// (for K).  One workgroup per 64 rows of one head.  The rounding to the E4M3 grid is
// done in fp64 (round to nearest even at the grid step of the value's binade), so
// that no intermediate fp32 rounding can move a value onto a midpoint; the result is
// on the grid, which the fp32 conversion then encodes exactly.
__device__ inline double e4m3_rne_f64(double y) {
  // no branch for zero: it falls on the subnormal grid and keeps its sign
  const double a = fabs(y);
  int E;
  frexp(a, &E);                                   // a in [2^(E-1), 2^E)
  const int step = a < 0x1.0p-6 ? -9 : (E - 1) - 3;  // grid step 2^step (subnormal below 2^-6)
  return copysign(ldexp(rint(ldexp(a, -step)), step), y);
}

__device__ inline int scale_exp_f64(double amax) {
  if (amax == 0.0) return 0;
  int E;
  const double m = frexp(amax, &E);
  return m <= 0.875 ? E - 9 : E - 8;
}

// x from the lane whose index differs in bit m (m = 1 or 2) within its quad of four lanes,
// by two DPP quad permutations of the halves (every lane of the quad is active)
__device__ inline double quad_xor_f64(double x, int m) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
  if (m == 1) {  // quad_perm [1, 0, 3, 2]
    lo = __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, true);
    hi = __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, true);
  } else {  // quad_perm [2, 3, 0, 1]
    lo = __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, true);
    hi = __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, true);
  }
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

template <int D, bool kPerRow>
__global__ __launch_bounds__(256) void pcast_prep_rot8(const uint16_t* __restrict__ x,
                                                       const signed char* __restrict__ signs,
                                                       uint8_t* __restrict__ codes, int* __restrict__ exps, int N,
                                                       int n_tiles) {
  // four lanes per row, each with V contiguous values: the transform's stages of
  // stride below V run in registers, the strides V and 2V across lanes (xor 1, 2)
  constexpr int V = D / 4;
  const int tid = threadIdx.x;
  const int r = tid / 4, part = tid % 4;
  // 64 rows of one head per workgroup; in a partial last block the rows past N are zeros
  // (they leave the block max unchanged): K codes are written for them (K's codes take
  // whole blocks per head), Q codes and exponents are not (Q keeps N rows per head)
  const int64_t bh = blockIdx.x / n_tiles;
  const int t = (int)(blockIdx.x % n_tiles);
  const bool exists = t * kKvBlock + r < N;
  const int64_t row = bh * N + (int64_t)t * kKvBlock + min(r, N - 1 - t * kKvBlock);  // source row
  const int64_t orow = kPerRow ? row : (int64_t)blockIdx.x * kKvBlock + r;          // code row
  const uint16_t* src = x + row * D + part * V;
  // the lane's V signs (16-byte aligned, V a multiple of 16) and values, all loads first
  i32x4_t sw[V / 16], xw[V / 8];
#pragma unroll
  for (int k = 0; k < V / 16; ++k) sw[k] = *reinterpret_cast<const i32x4_t*>(signs + part * V + k * 16);
#pragma unroll
  for (int k = 0; k < V / 8; ++k) xw[k] = exists ? *reinterpret_cast<const i32x4_t*>(src + k * 8) : i32x4_t{0, 0, 0, 0};
  double v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const uint32_t u = (uint32_t)xw[i / 8][(i % 8) / 2];
    const double f = (double)__builtin_bit_cast(float, (i & 1) ? (u & 0xFFFF0000u) : (u << 16));
    const int sgn = (int)(signed char)(((uint32_t)sw[i / 16][(i % 16) / 4] >> (8 * (i % 4))) & 0xFFu);
    v[i] = sgn < 0 ? -f : f;
  }
  // in-lane stages (natural, Sylvester order)
#pragma unroll
  for (int h = 1; h < V; h *= 2)
#pragma unroll
    for (int i = 0; i < V; ++i)
      if ((i & h) == 0) {
        const double a = v[i], c = v[i + h];
        v[i] = a + c;
        v[i + h] = a - c;
      }
  // cross-lane stages: the lower partner keeps the sum, the upper the difference
  // (o - v as o + (-v), the same rounding); the partner's value comes by a quad DPP move
#pragma unroll
  for (int m = 1; m <= 2; m *= 2) {
    const uint64_t flip = (part & m) != 0 ? 1ull << 63 : 0ull;  // the upper partner negates its own
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const double o = quad_xor_f64(v[i], m);
      v[i] = __builtin_bit_cast(double, __builtin_bit_cast(uint64_t, v[i]) ^ flip) + o;
    }
  }
  double mx = 0.0;
#pragma unroll
  for (int i = 0; i < V; ++i) mx = fmax(mx, fabs(v[i]));
  mx = fmax(mx, quad_xor_f64(mx, 1));
  mx = fmax(mx, quad_xor_f64(mx, 2));
  int e;
  if constexpr (kPerRow) {
    e = scale_exp_f64(mx);
    if (part == 0 && exists) exps[row] = e;
  } else {
    // the block's exponent from the max over its 64 rows
    __shared__ double rmax[kKvBlock];
    if (part == 0) rmax[r] = mx;
    __syncthreads();
    double bm = 0.0;
    for (int i = 0; i < kKvBlock; ++i) bm = fmax(bm, rmax[i]);
    e = scale_exp_f64(bm);
    if (tid == 0) exps[blockIdx.x] = e;
  }
  if (kPerRow && !exists) return;
  // the lane's V codes (16-byte aligned: the code buffer is, and D and V are multiples of 16)
  i32x4_t* dst = reinterpret_cast<i32x4_t*>(codes + orow * D + part * V);
#pragma unroll
  for (int c = 0; c < V / 16; ++c) {
    i32x4_t w;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float f[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) f[t] = (float)e4m3_rne_f64(ldexp(v[16 * c + 4 * k + t], -e));
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      w[k] = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], word, true);
    }
    dst[c] = w;
  }
}

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const void* vop;
  const float* bias;
  float* out;
  unsigned long long* stats;
  int B, Hq, Hkv, N;
  int order;
  float logit_scale;  // log2(e) / sqrt(d)
  float S;            // P-cast scale (1 in the bf16 path)
  float inv_S;        // 1/S: the conversion scale when S is a power of two
  float p_clamp;      // largest P kept before conversion when S > 448 (448/S)
  // FP8 logits: E4M3 codes of K ([B][Hkv][N][d] bytes) and the exponent of each key block;
  // with the rotation also the codes of Q ([B][Hq][N][d]) and the exponent of each row
  const uint8_t* k8;
  const int* kexp;
  const uint8_t* q8;
  const int* qexp;
  // per-row diagnostics [B][Hq][N], or null
  float* lse;
  float* lost;
  // decode with split KV: Nq query rows at the end of Nk keys, ranges of split_blocks
  // key blocks, partial results per (b, kv head, range, packed row)
  int Nq, Nk, n_split, split_blocks;
  float* part_a;          // [..][32][D] un-normalised accumulator
  float* part_ml;         // [..][32][2] running max (log2 units) and row sum
  unsigned int* part_cnt; // [..][32][2] non-sink pairs, zero codes
  // backward: raw V (bf16), dO (bf16), the forward's lse (natural units) and the row
  // dots D = dO . O; gradients (fp32)
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse_in;
  const float* dvec;      // -D = -(dO . O) per row
  const float* nls;       // -lse * sqrt(d) per row: lse in the logits' own units
  float* dq;
  float* dk;
  float* dv;
};

// How P becomes an MFMA operand.
enum PMode : int {
  kPow2 = 0,       // E4M3, S = 2^k <= 448: scaling inside the conversion (exact)
  kPow2Clamp = 1,  // E4M3, S = 2^k > 448: P clamped to 448/S first
  kMul = 2,        // E4M3, other S <= 448: fp32 multiply, then conversion
  kMulClamp = 3,   // E4M3, other S > 448: clamp, multiply, convert
  kBf16 = 4,       // no P-cast: P and V in bf16
};

// Convert 4 probabilities to 4 E4M3 codes in one word.
template <int kMode>
__device__ inline uint32_t cast4(const Params& p, float a, float b, float c, float d) {
  if constexpr (kMode == kPow2Clamp || kMode == kMulClamp) {
    const float lim = p.p_clamp;
    a = fminf(a, lim); b = fminf(b, lim); c = fminf(c, lim); d = fminf(d, lim);
  }
  if constexpr (kMode == kPow2 || kMode == kPow2Clamp) {
    // both halves of the word are written; its old contents (a's bits) are never read
    s16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(s16x2_t, a), a, b, p.inv_S, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c, d, p.inv_S, true);
    return __builtin_bit_cast(uint32_t, r);
  } else {
    const float S = p.S;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a * S, b * S, __builtin_bit_cast(int, a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c * S, d * S, w, true);
    return (uint32_t)w;
  }
}

// The P-cast conversion on its own, over a caller array of probabilities: four
// per lane through cast4<kMode>, the device code every attention kernel runs on P.
template <int kMode>
__global__ __launch_bounds__(256) void pcast_cast_probs(const Params p, const float4* __restrict__ src,
                                                         uint32_t* __restrict__ dst, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const float4 v = src[i];
    dst[i] = cast4<kMode>(p, v.x, v.y, v.z, v.w);
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// a in the low half, b in the high half, each rounded to nearest even (one
// v_cvt_pk_bf16_f32)
__device__ inline uint32_t cast2_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

typedef __attribute__((address_space(1))) const void global_cvoid;
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS: lane i writes
// lds + 16*i (global_load_lds_dwordx4; `lds` must be the same in every lane).
__device__ inline void load_to_lds16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((global_cvoid*)src, (lds_void*)lds, 16, 0, 0);
}

// The same through a buffer resource (buffer_load_dword* ... lds): base is
// wave-uniform, voff the lane's byte offset (below 2^31).  Unlike the global form,
// which the compiler must treat as a possible LDS access in flight (every later LDS
// read then waits for lgkmcnt(0)), this keeps its LDS waits exact.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ inline void buffer_to_lds16(__amdgpu_buffer_rsrc_t rs, int voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, 0, 0, 0);
}
__device__ inline void buffer_to_lds4(__amdgpu_buffer_rsrc_t rs, int voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 4, voff, 0, 0, 0);
}

// 4 bytes per lane from global memory straight into LDS (lane i writes lds + 4*i).
__device__ inline void load_to_lds4(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((global_cvoid*)src, (lds_void*)lds, 4, 0, 0);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

// An MFMA operand fragment of 8 bf16 read across the rows of a row-major LDS tile
// with two transposing reads (ds_read_b64_tr_b16): within each 16-lane group, lane
// i receives element (i % 4) of the 8-byte pieces addressed by lanes 4e + i / 4,
// e = 0..3, of its group.  Elements 0..3 come from the pieces at lo, 4..7 from hi.
__device__ inline bf16x8_t tr_frag(const uint8_t* lo, const uint8_t* hi) {
  const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)lo);
  const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)hi);
  const i32x4_t w = {__builtin_bit_cast(int, __builtin_shufflevector(a, a, 0, 1)),
                     __builtin_bit_cast(int, __builtin_shufflevector(a, a, 2, 3)),
                     __builtin_bit_cast(int, __builtin_shufflevector(b, b, 0, 1)),
                     __builtin_bit_cast(int, __builtin_shufflevector(b, b, 2, 3))};
  return __builtin_bit_cast(bf16x8_t, w);
}

// max over the two 32-lane halves (lane l and lane l ^ 32 hold the same query row)
__device__ inline float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}

// Sum over the 64 lanes of a wave, returned uniform: DPP row shifts leave each
// 16-lane row's total in its lane 15, the two row broadcasts carry them into lane 63.
__device__ inline unsigned int wave_sum(unsigned int x) {
  x += (unsigned int)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += (unsigned int)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += (unsigned int)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += (unsigned int)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += (unsigned int)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (unsigned int)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return (unsigned int)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ inline float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                                  false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// Workgroup -> (batch, head, 128-row block).  The hardware hands workgroup i
// to XCD i % 8; the remap gives each XCD a contiguous range of heads so that
// the K/V of a head are read into one XCD's L2, and within a head the
// longest (causal) row blocks start first.
__device__ inline void decode_block(int lin, int total, int n_rb, int Hq, bool causal, int& b, int& h,
                                    int& rb) {
  const int q = total / 8, r = total % 8;
  const int xcd = lin % 8, slot = lin / 8;
  const int v = (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
  const int hh = v / n_rb, rbi = v % n_rb;
  rb = causal ? n_rb - 1 - rbi : rbi;
  b = hh / Hq;
  h = hh % Hq;
}

template <bool kB, class T, class F>
struct Select {
  using type = T;
};
template <class T, class F>
struct Select<false, T, F> {
  using type = F;
};

template <int V>
struct BufIndex {
  static constexpr int value = V;
};

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time so
// that every register array index in f is a constant
template <class F, int... I>
__device__ __attribute__((always_inline)) inline void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}
template <int V>
using IC = std::integral_constant<int, V>;

// ---------------------------------------------------------------------------
// Attention kernel for the path without the P-cast (S = 0): P and V in bf16, P.V
// on v_mfma_f32_32x32x16_bf16.  Same tiling and staging as the FP8 kernel below,
// one step per block without its deferral.
// ---------------------------------------------------------------------------
template <int D, bool kCausal, bool kStats>
__global__ __launch_bounds__(kThreads, 2) void pcast_attn_fwd_bf16(const Params p) {
  using G = Geometry<D>;
  constexpr int kKRow = D * 2;                // bytes per K row
  constexpr int kVRow = kKvBlock * 2;         // bytes per V^T row (64 bf16 values)
  constexpr int kKTile = kKvBlock * kKRow;    // bytes of one K block
  constexpr int kVTile = D * kVRow;           // bytes of one V operand block
  using SK = Swizzle<kKRow>;
  using SV = Swizzle<kVRow>;
  constexpr int kKLoads = kKTile / (1024 * kWaves);  // 1 KB direct loads per wave and block
  constexpr int kVLoads = kVTile / (1024 * kWaves);
  static_assert(kKTile % (1024 * kWaves) == 0 && kVTile % (1024 * kWaves) == 0, "staging split");

  // one LDS object per staging buffer (see the FP8 kernel)
  __shared__ __attribute__((aligned(16))) uint8_t lds_k0[kKTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_k1[kKTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v0[kVTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v1[kVTile];
  __shared__ __attribute__((aligned(16))) float lds_b0[kKvBlock];
  __shared__ __attribute__((aligned(16))) float lds_b1[kKvBlock];
  __shared__ unsigned int lds_cnt[2][2];
  auto kbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_k1 : lds_k0; };
  auto vbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_v1 : lds_v0; };
  auto bbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_b1 : lds_b0; };

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int g = lane / 32, li = lane % 32;
  const int n_rb = (p.N + kBlockRows - 1) / kBlockRows;
  int b, h, rb;
  decode_block(blockIdx.x, n_rb * p.Hq * p.B, n_rb, p.Hq, kCausal, b, h, rb);
  const int hk = h / (p.Hq / p.Hkv);
  // key blocks; with N not a multiple of 64 the last one is partial: its keys past N get
  // a bias of -inf in LDS (probability 0, and not counted, as a sink would not be)
  const int n_tiles = (p.N + kKvBlock - 1) / kKvBlock, n_full = p.N / kKvBlock;
  const int row0 = rb * kBlockRows;
  const int wrow0 = row0 + wave * kRowsPerWave;  // first row of this wave
  const int myrow = wrow0 + li;
  const bool wave_active = wrow0 < p.N;  // rows past N (last row block) are computed, never stored
  const int t_last = kCausal ? min((row0 + kBlockRows - 1) / kKvBlock, n_tiles - 1) : n_tiles - 1;
  const int n_it = t_last + 1;
  const float c = p.logit_scale;

  if (kStats && tid < 4) lds_cnt[tid / 2][tid % 2] = 0;

  // Q operand (B of S^T = K Q^T): lane holds Q[myrow][s*16 + g*8 .. +8) for each step s.
  bf16x8_t qf[G::kQSteps];
  if (wave_active) {
    const uint16_t* qrow = p.q + (((int64_t)b * p.Hq + h) * p.N + min(myrow, p.N - 1)) * D + g * 8;
#pragma unroll
    for (int s = 0; s < G::kQSteps; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + s * 16);
  }

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k + ((int64_t)b * p.Hkv + hk) * p.N * D);
  const uint8_t* vbase = static_cast<const uint8_t*>(p.vop) + ((int64_t)b * p.Hkv + hk) * (int64_t)n_tiles * kVTile;
  int ksrc[kKLoads], vsrc[kVLoads];
#pragma unroll
  for (int i = 0; i < kKLoads; ++i) {
    const int pos = (wave * kKLoads + i) * 64 + lane, r = pos / SK::kChunks;
    ksrc[i] = r * kKRow + (((pos % SK::kChunks) ^ SK::key(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < kVLoads; ++i) {
    const int pos = (wave * kVLoads + i) * 64 + lane, r = pos / SV::kChunks;
    vsrc[i] = r * kVRow + (((pos % SV::kChunks) ^ SV::key(r)) << 4);
  }
  const bool with_bias = p.bias != nullptr;
  auto tile_of = [&](int it) __attribute__((always_inline)) { return p.order ? (t_last - it) : it; };
  auto visible = [&](int t) __attribute__((always_inline)) {
    return wave_active && (!kCausal || t * kKvBlock <= wrow0 + kRowsPerWave - 1);
  };
  auto load_k = [&](int t, int buf) __attribute__((always_inline)) {
    const uint8_t* ks = kbase + t * kKTile;
    if (t < n_full) {
#pragma unroll
      for (int i = 0; i < kKLoads; ++i) load_to_lds16(ks + ksrc[i], kbuf(buf) + (wave * kKLoads + i) * 1024);
    } else {
      // partial last block: rows past N read row N - 1 instead (their bias is -inf)
      const int last = (p.N - 1 - t * kKvBlock) * kKRow;  // byte offset of row N - 1 in the tile
#pragma unroll
      for (int i = 0; i < kKLoads; ++i)
        load_to_lds16(ks + min(ksrc[i], last + (ksrc[i] & (kKRow - 1))), kbuf(buf) + (wave * kKLoads + i) * 1024);
    }
  };
  // V of a block and its bias travel together
  auto load_v = [&](int t, int buf) __attribute__((always_inline)) {
    const uint8_t* vs = vbase + t * kVTile;
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) load_to_lds16(vs + vsrc[i], vbuf(buf) + (wave * kVLoads + i) * 1024);
    if (t < n_full) {
      if (with_bias && wave == 0) load_to_lds4(p.bias + t * kKvBlock + lane, bbuf(buf));
    } else if (wave == 0) {
      const int key = t * kKvBlock + lane;
      bbuf(buf)[lane] = key < p.N ? (with_bias ? p.bias[key] : 0.0f) : -INFINITY;
    }
  };
  auto wait_loads = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  const int xk = SK::key(li);  // rows li and li + 32 share the swizzle key
  auto issue_s = [&](int buf, f32x16_t(&sa)[2]) __attribute__((always_inline)) {
    const uint8_t* kl = kbuf(buf) + li * kKRow;
#pragma unroll
    for (int s = 0; s < G::kQSteps; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kl + kb * 32 * kKRow + (((2 * s + g) ^ xk) << 4));
        sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], s == 0 ? f32x16_t{} : sa[kb], 0, 0, 0);
      }
    }
  };
  f32x16_t oacc[G::kDTiles];
#pragma unroll
  for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
  f32x16_t sacc[2];  // logits (then probabilities) of the block being processed
  float m_run = -INFINITY, l_run = 0.0f;
  unsigned int cnt_tot = 0, cnt_zero = 0;

  // Softmax of a block, in place, with the causal mask and the bias where present.
  auto softmax = [&](f32x16_t(&sa)[2], int key0, bool diag, bool has_bias, int buf)
      __attribute__((always_inline)) -> float {
    float bk[32];
    if (has_bias) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(bbuf(buf) + slot_key(g, 4 * q));
        bk[4 * q] = v.x; bk[4 * q + 1] = v.y; bk[4 * q + 2] = v.z; bk[4 * q + 3] = v.w;
      }
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int kj = slot_key(g, j);
      float xj = has_bias ? fmaf(sa[j / 16][j % 16], c, bk[j] * kLog2e) : sa[j / 16][j % 16] * c;
      if (diag && key0 + kj > myrow) xj = -INFINITY;
      sa[j / 16][j % 16] = xj;
    }
    float mx = sa[0][0];
#pragma unroll
    for (int j = 1; j < 32; ++j) mx = fmaxf(mx, sa[j / 16][j % 16]);
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float pj = __builtin_amdgcn_exp2f(sa[j / 16][j % 16] - m_use);
      sa[j / 16][j % 16] = pj;
      ps[j % 4] += pj;
    }
    l_run = l_run * alpha + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
    m_run = m_new;
    if constexpr (kStats) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int kj = slot_key(g, j);
        const bool vis_j = !kCausal || key0 + kj <= myrow;
        const bool nonsink = !has_bias || bk[j] == 0.0f;
        // the bf16 code of P is zero only when P itself rounds to zero
        const bool z = (__builtin_bit_cast(uint16_t, (__bf16)sa[j / 16][j % 16]) & 0x7FFFu) == 0;
        cnt_tot += (vis_j && nonsink);
        cnt_zero += (vis_j && nonsink && z);
      }
    }
    return alpha;
  };

  auto step = [&](int it, auto cur_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value, nxt = cur ^ 1;
    const int t = tile_of(it);
    // K of block it+2 replaces K of block it (read during step it-1); V and bias of
    // block it+1 replace those of block it-1.  Both land while this step computes.
    if (it + 2 < n_it) load_k(tile_of(it + 2), cur);
    if (it + 1 < n_it) load_v(tile_of(it + 1), nxt);
    const bool vis = visible(t);
    const bool vis1 = it + 1 < n_it && visible(tile_of(it + 1));
    if (vis) {
      const int key0 = t * kKvBlock;
      const bool diag = kCausal && (key0 + kKvBlock - 1 > wrow0);
      const bool has_bias = (with_bias || t >= n_full) && __builtin_amdgcn_ballot_w64(bbuf(cur)[lane] != 0.0f) != 0;
      const float alpha = softmax(sacc, key0, diag, has_bias, cur);
      uint32_t pw[16];
#pragma unroll
      for (int w = 0; w < 16; ++w) pw[w] = cast2_bf16(sacc[w / 8][(2 * w) % 16], sacc[w / 8][(2 * w + 1) % 16]);
      // O^T = alpha O^T, skipped when alpha == 1 in every lane (an exact no-op)
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      }
      if (vis1) issue_s(nxt, sacc);
      // O^T += V^T P^T: four k-steps of 16 keys per 32-column tile
      const uint8_t* vl = vbuf(cur) + li * kVRow;
      const int xv = SV::key(li);
#pragma unroll
      for (int dt = 0; dt < G::kDTiles; ++dt) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vl + dt * 32 * kVRow + (((4 * g + s) ^ xv) << 4));
          const i32x4_t bw = {(int)pw[4 * s], (int)pw[4 * s + 1], (int)pw[4 * s + 2], (int)pw[4 * s + 3]};
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bw), oacc[dt], 0, 0, 0);
        }
      }
    } else if (vis1) {
      issue_s(nxt, sacc);
    }
    wait_loads();
    __syncthreads();
  };

  // prologue: K, V and bias of the first block, K of the second; logits of the first block
  load_k(tile_of(0), 0);
  load_v(tile_of(0), 0);
  if (n_it > 1) load_k(tile_of(1), 1);
  wait_loads();
  __syncthreads();
  if (visible(tile_of(0))) issue_s(0, sacc);
  // step 0 reloads K buffer 0: every wave must have read block 0's K first
  __syncthreads();
  for (int it = 0; it < n_it; it += 2) {
    step(it, BufIndex<0>{});
    if (it + 1 < n_it) step(it + 1, BufIndex<1>{});
  }

  // ---- epilogue: O = A / l (S = 1 on this path) ----
  if (myrow < p.N) {
    const float inv = 1.0f / (p.S * halves_sum(l_run));
    float* orow = p.out + (((int64_t)b * p.Hq + h) * p.N + myrow) * D;
#pragma unroll
    for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 v;
        v.x = oacc[dt][r4 * 4 + 0] * inv;
        v.y = oacc[dt][r4 * 4 + 1] * inv;
        v.z = oacc[dt][r4 * 4 + 2] * inv;
        v.w = oacc[dt][r4 * 4 + 3] * inv;
        *reinterpret_cast<float4*>(orow + dt * 32 + r4 * 8 + g * 4) = v;
      }
  }
  if constexpr (kStats) {
    const bool counted = myrow < p.N;
    const unsigned int a = wave_sum(counted ? cnt_tot : 0u), z = wave_sum(counted ? cnt_zero : 0u);
    if (lane == 0 && wave_active) {
      atomicAdd(&lds_cnt[wave / 2][0], a);
      atomicAdd(&lds_cnt[wave / 2][1], z);
    }
    __syncthreads();
    if (tid < 2) {
      const int r64 = row0 / kKvBlock + tid;  // 64-row block index
      if (r64 * kKvBlock < p.N) {
        unsigned long long* st = p.stats + 2 * (((int64_t)b * p.Hq + h) * n_tiles + r64);
        st[0] = lds_cnt[tid][0];
        st[1] = lds_cnt[tid][1];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Attention kernel for the FP8 P-cast modes, software-pipelined by one block:
// step j exponentiates and casts block j (its logits sit in one of two logit
// buffers) while the same wave's MFMAs form block j+1's logits in the other
// buffer and accumulate block j-1's P.V, deferred by one step (the rescale by
// block j-1's alpha comes first).  The three streams are independent, so the
// MFMAs interleave with the exponentials inside one basic block.
// ---------------------------------------------------------------------------
// Several configurations of one forward in one launch: the cells share Q, K and the V
// operand copy, each has its own bias, scale, key-block order, output and counters.
// The table travels by value in the kernel arguments.
// Configurations per launch: the table travels in the kernel arguments (4 KiB with
// the Params); 1/S and the clamp 448/S are formed in the kernel with the same
// correctly rounded division as on the host.
constexpr int kMaxCells = 112;
struct Cells {
  const float* bias[kMaxCells];
  float* out[kMaxCells];
  unsigned long long* stats[kMaxCells];
  float S[kMaxCells];
  int order[kMaxCells];
  int n;
};
static_assert(sizeof(Cells) + sizeof(Params) <= 4096, "kernel arguments above 4 KiB");
struct NoCells {};

// kStats: 0 = no counting; 1 = underflow counters; 2 = counters (if p.stats) and the
// per-row log-sum-exp and lost non-sink mass (every block then takes the sequential step).
// kQ8: 0 = bf16 logits; 1 = FP8 logits, Q rounded here per row; 2 = FP8 logits of the
// rotated Q and K, both as codes from the pre-pass.
// kMulti: the grid covers cells.n configurations (an outer batch dimension), each
// workgroup taking its cell's bias, scale, order, output and counters from the table.
template <int D, int kMode, bool kCausal, int kStats, int kQ8, bool kMulti = false>
__global__ __launch_bounds__(kThreads, 2) void pcast_attn_fwd_fp8(
    const Params p0, const typename Select<kMulti, Cells, NoCells>::type cells) {
  static_assert(kMode != kBf16, "FP8 modes only");
  static_assert(!kMulti || (kStats < 2 && kQ8 == 0), "configuration cells: bf16 logits, no row diagnostics");
  Params p = p0;
  constexpr bool kDiag = kStats == 2;
  using G = Geometry<D>;
  // kQ8: Q and K as E4M3 codes, logits on the FP8 MFMA (K = 64 per step), else bf16
  constexpr int kKRow = kQ8 ? D : D * 2;      // bytes per K row
  constexpr int kSSteps = kQ8 ? D / 64 : G::kQSteps;  // logit MFMA k-steps per 32-key half
  using KFrag = typename Select<kQ8 != 0, i32x8_t, bf16x8_t>::type;  // one operand fragment
  constexpr int kVRow = kKvBlock;             // bytes per V^T row (64 E4M3 codes)
  constexpr int kKTile = kKvBlock * kKRow;    // bytes of one K block
  constexpr int kVTile = D * kVRow;           // bytes of one V operand block
  using SK = Swizzle<kKRow>;
  using SV = Swizzle<kVRow>;
  constexpr int kKLoads = kKTile / (1024 * kWaves);  // 1 KB direct loads per wave and block
  constexpr int kVLoads = kVTile / (1024 * kWaves);
  static_assert(kKTile % (1024 * kWaves) == 0 && kVTile % (1024 * kWaves) == 0, "staging split");

  // Each staging buffer is its own LDS object, so the compiler can tell that the
  // direct loads into one buffer never alias reads of the other and does not make
  // those reads wait for the loads in flight.
  __shared__ __attribute__((aligned(16))) uint8_t lds_k0[kKTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_k1[kKTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v0[kVTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v1[kVTile];
  __shared__ __attribute__((aligned(16))) float lds_b0[kKvBlock];
  __shared__ __attribute__((aligned(16))) float lds_b1[kKvBlock];
  __shared__ unsigned int lds_cnt[2][2];
  // buffer indices are compile-time constants wherever these are called
  auto kbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_k1 : lds_k0; };
  auto vbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_v1 : lds_v0; };
  auto bbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_b1 : lds_b0; };

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int g = lane / 32, li = lane % 32;
  const int n_rb = (p.N + kBlockRows - 1) / kBlockRows;
  int b, h, rb;
  if constexpr (kMulti) {
    // cells are the innermost index of the (batch, head) range an XCD takes: the cells
    // of a head follow one another, so its K and V stay in that XCD's L2
    decode_block(blockIdx.x, n_rb * p.Hq * p.B * cells.n, n_rb, p.Hq, kCausal, b, h, rb);
    const int hh = b * p.Hq + h;
    const int cell = hh % cells.n, bh = hh / cells.n;
    b = bh / p.Hq;
    h = bh % p.Hq;
    p.bias = cells.bias[cell];
    p.out = cells.out[cell];
    p.stats = cells.stats[cell];
    p.S = cells.S[cell];
    p.inv_S = 1.0f / p.S;
    p.p_clamp = 448.0f / p.S;
    p.order = cells.order[cell];
  } else {
    decode_block(blockIdx.x, n_rb * p.Hq * p.B, n_rb, p.Hq, kCausal, b, h, rb);
  }
  const int hk = h / (p.Hq / p.Hkv);
  // key blocks; with N not a multiple of 64 the last one is partial (keys past N masked)
  const int n_tiles = (p.N + kKvBlock - 1) / kKvBlock, n_full = p.N / kKvBlock;
  const int row0 = rb * kBlockRows;
  const int wrow0 = row0 + wave * kRowsPerWave;  // first row of this wave
  const int myrow = wrow0 + li;
  const bool wave_active = wrow0 < p.N;
  const bool row_valid = myrow < p.N;  // rows past N (last row block) are computed, never stored
  const int t_last = kCausal ? min((row0 + kBlockRows - 1) / kKvBlock, n_tiles - 1) : n_tiles - 1;
  const int n_it = t_last + 1;
  // log2(e)/sqrt(d); with FP8 logits times 2^(e_row + e_block) of the row's and the
  // key block's scales (exact), set per block
  float c = p.logit_scale;

  if (kStats && tid < 4) lds_cnt[tid / 2][tid % 2] = 0;

  // Q operand (B of S^T = K Q^T): lane holds Q[myrow][s*16 + g*8 .. +8) for each step s
  // (bf16), or the E4M3 codes of Q[myrow][s*64 + g*32 .. +32) * 2^-e_row (FP8, the row's
  // scale from the max over both lane halves).  The K fragments take the same d order,
  // so slot k of the two operands holds the same d.
  KFrag qf[kSSteps];
  float c_row = p.logit_scale;
  if (wave_active) {
    const int64_t row = ((int64_t)b * p.Hq + h) * p.N + min(myrow, p.N - 1);
    if constexpr (kQ8 == 2) {
      // the pre-pass's codes of the rotated row; the rotation scales Q K^T by d
      const uint8_t* qrow = p.q8 + row * D + g * 32;
#pragma unroll
      for (int s = 0; s < kSSteps; ++s) {
        const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(qrow + s * 64);
        const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(qrow + s * 64 + 16);
        qf[s] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      c_row = ldexpf(p.logit_scale, p.qexp[row] - (D == 64 ? 6 : 7));
    } else if constexpr (kQ8 == 1) {
      const uint16_t* qrow = p.q + row * D + g * 32;
      i32x4_t w[kSSteps][4];
      uint32_t m = 0;
#pragma unroll
      for (int s = 0; s < kSSteps; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          w[s][t] = *reinterpret_cast<const i32x4_t*>(qrow + s * 64 + t * 8);
          m = max(m, absmax8(w[s][t]));
        }
      m = max(m, (uint32_t)__shfl_xor((int)m, 32));
      const int e = scale_exp(m);
#pragma unroll
      for (int s = 0; s < kSSteps; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          int lo, hi;
          codes8(w[s][t], e, lo, hi);
          qf[s][2 * t] = lo;
          qf[s][2 * t + 1] = hi;
        }
      c_row = ldexpf(p.logit_scale, e);
    } else {
      const uint16_t* qrow = p.q + row * D + g * 8;
#pragma unroll
      for (int s = 0; s < kSSteps; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + s * 16);
    }
  }

  // FP8 K codes are laid out in whole key blocks per head
  const uint8_t* kbase = kQ8 ? p.k8 + ((int64_t)b * p.Hkv + hk) * n_tiles * kKTile
                             : reinterpret_cast<const uint8_t*>(p.k + ((int64_t)b * p.Hkv + hk) * p.N * D);
  const uint8_t* vbase = static_cast<const uint8_t*>(p.vop) + ((int64_t)b * p.Hkv + hk) * (int64_t)n_tiles * kVTile;

  // Each lane's source offsets for the direct loads: lane i of load j of wave w fills
  // LDS chunk position (w * loads + j) * 64 + i, which holds logical chunk
  // position ^ key(row) of that row.
  int ksrc[kKLoads], vsrc[kVLoads];
#pragma unroll
  for (int i = 0; i < kKLoads; ++i) {
    const int pos = (wave * kKLoads + i) * 64 + lane, r = pos / SK::kChunks;
    ksrc[i] = r * kKRow + (((pos % SK::kChunks) ^ SK::key(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < kVLoads; ++i) {
    const int pos = (wave * kVLoads + i) * 64 + lane, r = pos / SV::kChunks;
    vsrc[i] = r * kVRow + (((pos % SV::kChunks) ^ SV::key(r)) << 4);
  }
  const bool with_bias = p.bias != nullptr;
  auto tile_of = [&](int it) __attribute__((always_inline)) { return p.order ? (t_last - it) : it; };
  auto visible = [&](int t) __attribute__((always_inline)) {
    return wave_active && (!kCausal || t * kKvBlock <= wrow0 + kRowsPerWave - 1);
  };
  // The LDS destination of a direct load is a wave-uniform register (M0): form this
  // wave's offset once per load group as a scalar, so that no load waits on a
  // vector-to-scalar move.
  auto load_k = [&](int t, int buf) __attribute__((always_inline)) {
    const uint8_t* ks = kbase + t * kKTile;
    const int dst = __builtin_amdgcn_readfirstlane(wave * kKLoads * 1024);
    if (t < n_full) {
#pragma unroll
      for (int i = 0; i < kKLoads; ++i) load_to_lds16(ks + ksrc[i], kbuf(buf) + dst + i * 1024);
    } else {
      // partial last block: rows past N read row N - 1 instead (their logits are masked)
      const int last = (p.N - 1 - t * kKvBlock) * kKRow;  // byte offset of row N - 1 in the tile
#pragma unroll
      for (int i = 0; i < kKLoads; ++i)
        load_to_lds16(ks + min(ksrc[i], last + (ksrc[i] & (kKRow - 1))), kbuf(buf) + dst + i * 1024);
    }
  };
  auto load_v = [&](int t, int buf) __attribute__((always_inline)) {
    const uint8_t* vs = vbase + t * kVTile;
    const int dst = __builtin_amdgcn_readfirstlane(wave * kVLoads * 1024);
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) load_to_lds16(vs + vsrc[i], vbuf(buf) + dst + i * 1024);
  };
  // bias of key min(j, N - 1): keys past N take the last key's value (masked anyway)
  auto bias_at = [&](int t) __attribute__((always_inline)) { return p.bias + min(t * kKvBlock + lane, p.N - 1); };
  auto load_b = [&](int t, int buf) __attribute__((always_inline)) {
    if (with_bias && wave == 0) load_to_lds4(bias_at(t), bbuf(buf));
  };
  auto wait_loads = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // S^T = K Q^T for the key block in K buffer `buf`: two 32-key halves, fp32 accumulation
  const int xk = SK::key(li);  // rows li and li + 32 share the swizzle key
  // The lane's byte offset of each K chunk it reads within a tile (row li, swizzled
  // chunk), computed once; the empty asm keeps the compiler from splitting it again
  // into a row part and a chunk part, so that a read is this register plus an
  // immediate (buffer, 32-key half) and needs no add.
  constexpr int kKChunks = kQ8 ? 2 * kSSteps : kSSteps;
  int koff[kKChunks];
#pragma unroll
  for (int i = 0; i < kKChunks; ++i) {
    const int chunk = kQ8 ? (4 * (i / 2) + 2 * g + i % 2) : (2 * i + g);
    koff[i] = li * kKRow + ((chunk ^ xk) << 4);
    asm volatile("" : "+v"(koff[i]));
  }
  // K fragment of 32-key half kb and k-step s from K buffer `buf`
  auto kread = [&](int buf, int kb, int s) __attribute__((always_inline)) -> KFrag {
    const uint8_t* kl = kbuf(buf) + kb * 32 * kKRow;
    if constexpr (kQ8 != 0) {
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(kl + koff[2 * s]);
      const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(kl + koff[2 * s + 1]);
      return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return *reinterpret_cast<const bf16x8_t*>(kl + koff[s]);
    }
  };
  // the same for the two V chunks a lane reads per 32-column tile (row li of the tile)
  int voff[2];
  {
    const int xv = SV::key(li);  // rows dt*32 + li share the swizzle key
    voff[0] = li * kVRow + (((2 * g) ^ xv) << 4);
    voff[1] = li * kVRow + (((2 * g + 1) ^ xv) << 4);
    asm volatile("" : "+v"(voff[0]));
    asm volatile("" : "+v"(voff[1]));
  }
  auto vread = [&](int buf, int dt) __attribute__((always_inline)) -> i32x8_t {
    const uint8_t* vl = vbuf(buf) + dt * 32 * kVRow;
    const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(vl + voff[0]);
    const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(vl + voff[1]);
    return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto smma = [&](const KFrag& a, int s, const f32x16_t& acc) __attribute__((always_inline)) -> f32x16_t {
    if constexpr (kQ8 != 0) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[s], acc, 0, 0, 0, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], acc, 0, 0, 0);
  };
  auto issue_s = [&](int buf, f32x16_t(&sa)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kSSteps; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sa[kb] = smma(kread(buf, kb, s), s, s == 0 ? f32x16_t{} : sa[kb]);
    }
  };
  f32x16_t oacc[G::kDTiles];
#pragma unroll
  for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
  // O^T += V8^T P8^T for the V block in V buffer `buf`
  auto accumulate = [&](int buf, const i32x8_t& pb) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < G::kDTiles; ++dt)
      oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vread(buf, dt), pb, oacc[dt], 0, 0, 0, 0, 0, 0);
  };
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
    // alpha == 1 in every lane: an exact no-op, skipped
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
  };

  f32x16_t sacc[2];  // logits of the block being processed (two 32-key halves)
  i32x8_t pbuf[2];   // E4M3 codes of blocks of even and odd step index
  float m_run = -INFINITY, l_run = 0.0f;
  float alpha_pend = 1.0f;  // rescale owed before the pending P.V
  bool pend = false;        // block j-1's P.V is still to be accumulated
  unsigned int cnt_tot = 0, cnt_zero = 0, cnt_nz_fast = 0, n_fast = 0;
  // row diagnostics, rescaled like l: un-cast P of non-sink keys, and of those whose code is 0
  float l_ns = 0.0f, l_lost = 0.0f;

  // max of a block's raw logits (four max3 chains, then a tree; both lane halves)
  auto block_max = [&](f32x16_t(&sa)[2]) __attribute__((always_inline)) -> float {
    float m4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m4[q] = fmaxf(sa[q / 2][(q % 2) * 8], sa[q / 2][(q % 2) * 8 + 1]);
#pragma unroll
      for (int r = 2; r < 8; r += 2)
        m4[q] = fmaxf(fmaxf(m4[q], sa[q / 2][(q % 2) * 8 + r]), sa[q / 2][(q % 2) * 8 + r + 1]);
    }
    return halves_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
  };
  // Softmax and P-cast of a block with no mask and no sink: the max of the raw
  // logits gives the max of s*c (c > 0), and exp2(s*c - m') is one fma and one exp2.
  auto softmax_fast = [&](f32x16_t(&sa)[2], i32x8_t& pb) __attribute__((always_inline)) -> float {
    const float mx = block_max(sa);
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float neg = -m_new;
    float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float pj = __builtin_amdgcn_exp2f(fmaf(sa[j / 16][j % 16], c, neg));
      sa[j / 16][j % 16] = pj;
      ps[j % 4] += pj;
    }
    const float bsum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    l_run = l_run * alpha + bsum;
    m_run = m_new;
#pragma unroll
    for (int w = 0; w < 8; ++w)
      pb[w] = (int)cast4<kMode>(p, sa[w / 4][4 * (w % 4)], sa[w / 4][4 * (w % 4) + 1], sa[w / 4][4 * (w % 4) + 2],
                                sa[w / 4][4 * (w % 4) + 3]);
    if constexpr (kDiag) {  // every key visible and non-sink; summed in the order of bsum
      float lo[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 32; ++j)
        lo[j % 4] += (((uint32_t)pb[j / 4] >> (8 * (j % 4))) & 0xFFu) == 0 ? sa[j / 16][j % 16] : 0.0f;
      l_ns = l_ns * alpha + bsum;
      l_lost = l_lost * alpha + ((lo[0] + lo[1]) + (lo[2] + lo[3]));
    }
    return alpha;
  };
  // bias of this lane's 32 keys from the staged block: slots 4q..4q+3 are 4 consecutive keys
  auto lane_bias = [&](int buf, float (&bk)[32]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(bbuf(buf) + slot_key(g, 4 * q));
      bk[4 * q] = v.x; bk[4 * q + 1] = v.y; bk[4 * q + 2] = v.z; bk[4 * q + 3] = v.w;
    }
  };
  // Softmax and P-cast of a block with a causal mask or a sink bias, in place.
  auto softmax_general = [&](f32x16_t(&sa)[2], i32x8_t& pb, int key0, bool diag, bool has_bias, int buf)
      __attribute__((always_inline)) -> float {
    float bk[32];
    if (has_bias) lane_bias(buf, bk);
    // keys past the row's position (causal diagonal) or past N (a partial last block)
    const bool masked = diag || key0 + kKvBlock > p.N;
    const int kmax = min(diag ? myrow - key0 : kKvBlock - 1, p.N - 1 - key0);  // last visible key
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int kj = slot_key(g, j);
      float xj = has_bias ? fmaf(sa[j / 16][j % 16], c, bk[j] * kLog2e) : sa[j / 16][j % 16] * c;
      if (masked && kj > kmax) xj = -INFINITY;
      sa[j / 16][j % 16] = xj;
    }
    const float m_new = fmaxf(m_run, block_max(sa));
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float pj = __builtin_amdgcn_exp2f(sa[j / 16][j % 16] - m_use);
      sa[j / 16][j % 16] = pj;
      ps[j % 4] += pj;
    }
    l_run = l_run * alpha + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
    m_run = m_new;
#pragma unroll
    for (int w = 0; w < 8; ++w)
      pb[w] = (int)cast4<kMode>(p, sa[w / 4][4 * (w % 4)], sa[w / 4][4 * (w % 4) + 1], sa[w / 4][4 * (w % 4) + 2],
                                sa[w / 4][4 * (w % 4) + 3]);
    if constexpr (kDiag) {  // masked keys have P = 0 and add nothing
      float lo = 0.0f, ns = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const bool nonsink = has_bias ? bk[j] == 0.0f : true;
        const bool zero = (((uint32_t)pb[j / 4] >> (8 * (j % 4))) & 0xFFu) == 0;
        const float pj = sa[j / 16][j % 16];
        ns += nonsink ? pj : 0.0f;
        lo += (nonsink && zero) ? pj : 0.0f;
      }
      l_ns = l_ns * alpha + ns;
      l_lost = l_lost * alpha + lo;
    }
    if constexpr (kStats) {
      if (has_bias) {
        // per key: visible, non-sink, code zero
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const int kj = slot_key(g, j);
          const bool vis = (!kCausal || key0 + kj <= myrow) && key0 + kj < p.N;
          const bool nonsink = bk[j] == 0.0f;
          const bool z = (((uint32_t)pb[j / 4] >> (8 * (j % 4))) & 0xFFu) == 0;
          cnt_tot += (vis && nonsink);
          cnt_zero += (vis && nonsink && z);
        }
      } else {
        // causal mask and / or the end of the sequence.  The lane's 32 keys are eight
        // runs of four consecutive keys starting at h*32 + q*8 + g*4; the visible ones
        // are those below lim.  Masked keys have P = 0, whose code is 0, so the zero
        // codes among the visible keys are all zero codes minus the masked keys.
        const int lim = (kCausal ? min(myrow + 1, p.N) : p.N) - key0;  // keys below lim are visible
        int vis = 0;
#pragma unroll
        for (int run = 0; run < 8; ++run) vis += min(max(lim - ((run / 4) * 32 + (run % 4) * 8 + g * 4), 0), 4);
        unsigned int nz = 0;
#pragma unroll
        for (int w = 0; w < 8; ++w) nz = __builtin_amdgcn_msad_u8((uint32_t)pb[w] | 0x80808080u, (uint32_t)pb[w], nz);
        const int zeros = 32 - (int)(nz >> 7);
        cnt_tot += vis;
        cnt_zero += zeros - (32 - vis);
      }
    }
    return alpha;
  };
  // non-zero codes of a block where every pair is visible and non-sink: v_msad_u8
  // sums |(w | 0x80808080) - w| = 0x80 over the bytes where w is non-zero, so the
  // accumulator holds 128 times the count
  auto count_fast = [&](const i32x8_t& pb) __attribute__((always_inline)) {
    ++n_fast;
#pragma unroll
    for (int w = 0; w < 8; ++w)
      cnt_nz_fast = __builtin_amdgcn_msad_u8((uint32_t)pb[w] | 0x80808080u, (uint32_t)pb[w], cnt_nz_fast);
  };

  // Step j: block j in buffers cur = j % 2 (its logits, codes, V and bias), blocks
  // j-1 and j+1 in nxt.
  // FP8 logits: exponent of each key block's scale, read one step ahead
  const int* kexp_head = kQ8 ? p.kexp + ((int64_t)b * p.Hkv + hk) * n_tiles : nullptr;
  int ke_next = kQ8 ? kexp_head[tile_of(0)] : 0;
  // the lane's bias value in the block the next step processes (0 without a bias), read
  // from global memory one step ahead: the step's fast / general decision then waits
  // for no LDS read
  float bias_next = with_bias ? *bias_at(tile_of(0)) : 0.0f;

  auto step = [&](int it, auto cur_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value, nxt = cur ^ 1;
    const int t = tile_of(it);
    if constexpr (kQ8 != 0) {
      c = ldexpf(c_row, ke_next);
      if (it + 1 < n_it) ke_next = kexp_head[tile_of(it + 1)];
    }
    // K of block j+2 replaces K of block j (read during step j-1); V of block j
    // replaces V of block j-2 (read during step j-1); bias of block j+1 replaces
    // that of block j-1.  All land before the barrier that ends this step.
    if (it + 2 < n_it) load_k(tile_of(it + 2), cur);
    load_v(t, cur);
    if (it + 1 < n_it) load_b(tile_of(it + 1), nxt);
    const bool vis = visible(t);
    const bool vis1 = it + 1 < n_it && visible(tile_of(it + 1));
    const int key0 = t * kKvBlock;
    const bool diag = kCausal && (key0 + kKvBlock - 1 > wrow0);
    const bool has_bias = with_bias && __builtin_amdgcn_ballot_w64(bias_next != 0.0f) != 0;
    if (with_bias && it + 1 < n_it) bias_next = *bias_at(tile_of(it + 1));
    const bool fast = vis && !diag && !has_bias && t < n_full;
    if (!kDiag && fast && pend && vis1) {
      // Steady state: the step's MFMAs (20 at d = 128), each in a chunk of its own
      // with the fragment read two MFMAs ahead and a slice of VALU work that does
      // not depend on any MFMA in flight; sched_barrier fences keep the chunks in
      // this order.
      //   A: block j-1's P.V      | max, alpha, first half's exponentials and casts
      //   B: block j+1's logits, first half (over block j's, already cast)
      //                           | second half's exponentials and casts
      //   C: second half          | counters
      // The rescale owed by block j-1 comes first, skipped when no row's max grew.
      rescale(alpha_pend);
      i32x8_t& pb = pbuf[cur];
      auto vfrag = [&](int dt) __attribute__((always_inline)) { return vread(nxt, dt); };
      auto kfrag = [&](int f) __attribute__((always_inline)) {  // f = half * kSSteps + step
        return kread(nxt, f / kSSteps, f % kSSteps);
      };
      auto pv = [&](int dt, const i32x8_t& a) __attribute__((always_inline)) {
        oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pbuf[nxt], oacc[dt], 0, 0, 0, 0, 0, 0);
      };
      auto smfma = [&](int f, const KFrag& a) __attribute__((always_inline)) {
        const int hh = f / kSSteps, st = f % kSSteps;
        sacc[hh] = smma(a, st, st == 0 ? f32x16_t{} : sacc[hh]);
      };
      constexpr int kS = 2 * kSSteps;  // logit MFMAs
      i32x8_t vf[G::kDTiles];
      KFrag kf[kS];
      float m4[4], ps[4];
      auto chain = [&](int q) __attribute__((always_inline)) {
        m4[q] = fmaxf(sacc[q / 2][(q % 2) * 8], sacc[q / 2][(q % 2) * 8 + 1]);
#pragma unroll
        for (int r = 2; r < 8; r += 2)
          m4[q] = fmaxf(fmaxf(m4[q], sacc[q / 2][(q % 2) * 8 + r]), sacc[q / 2][(q % 2) * 8 + r + 1]);
      };
      float m_new = 0.0f, alpha = 1.0f, neg = 0.0f;
      auto expo = [&](int hh, int r) __attribute__((always_inline)) {
        const float pj = __builtin_amdgcn_exp2f(fmaf(sacc[hh][r], c, neg));
        sacc[hh][r] = pj;
        if (hh == 0 && r < 4) ps[r] = pj;  // the first four start the partial sums
        else ps[r % 4] += pj;
      };
      auto cast = [&](int w) __attribute__((always_inline)) {  // codes of slots 4w..4w+3
        const int hh = w / 4, r = 4 * (w % 4);
        pb[w] = (int)cast4<kMode>(p, sacc[hh][r], sacc[hh][r + 1], sacc[hh][r + 2], sacc[hh][r + 3]);
      };
#define PCAST_FENCE __builtin_amdgcn_sched_barrier(0)
      // operand fragments run kAhead MFMAs ahead: MFMA i (P.V tiles first, then the
      // logit halves) takes fragment i
      constexpr int kAhead = 4;
      constexpr int kM = G::kDTiles + kS;
      auto fetch = [&](int i) __attribute__((always_inline)) {
        if (i < G::kDTiles) vf[i] = vfrag(i);
        else if (i < kM) kf[i - G::kDTiles] = kfrag(i - G::kDTiles);
      };
#pragma unroll
      for (int i = 0; i < kAhead; ++i) fetch(i);
      PCAST_FENCE;
      // ---- A: P.V MFMAs, the VALU work in 25 units (four max chains, the max
      // itself and alpha, 16 exponentials, four casts) spread evenly over them ----
      constexpr int kAUnits = 4 + 1 + 16 + 4;
      auto aunit = [&](int u) __attribute__((always_inline)) {
        if (u < 4) {
          chain(u);
        } else if (u == 4) {
          const float mx = halves_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
          m_new = fmaxf(m_run, mx * c);
          alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          neg = -m_new;
        } else if (u < 21) {
          expo(0, u - 5);
        } else {
          cast(u - 21);
        }
      };
#pragma unroll
      for (int i = 0; i < G::kDTiles; ++i) {
        pv(i, vf[i]);
        fetch(kAhead + i);
#pragma unroll
        for (int u = i * kAUnits / G::kDTiles; u < (i + 1) * kAUnits / G::kDTiles; ++u) aunit(u);
        PCAST_FENCE;
      }
      // ---- B and C ----
#pragma unroll
      for (int f = 0; f < kS; ++f) {
        smfma(f, kf[f]);
        fetch(G::kDTiles + f + kAhead);
        if (f < kSSteps) {
          // second half's exponentials, 16 over kSSteps chunks, each group of four
          // cast as soon as it is complete
          constexpr int kPer = 16 / kSSteps;
#pragma unroll
          for (int r = 0; r < kPer; ++r) expo(1, f * kPer + r);
#pragma unroll
          for (int w = f * kPer / 4; w < (f + 1) * kPer / 4; ++w) cast(4 + w);
        } else {
          const int k = f - kSSteps;
          if constexpr (kStats) {
            constexpr int kW = 8 / kSSteps;
#pragma unroll
            for (int e = 0; e < kW; ++e) {
              const int w = k * kW + e;
              cnt_nz_fast = __builtin_amdgcn_msad_u8((uint32_t)pb[w] | 0x80808080u, (uint32_t)pb[w], cnt_nz_fast);
            }
          }
        }
        PCAST_FENCE;
      }
#undef PCAST_FENCE
      if constexpr (kStats) ++n_fast;
      l_run = l_run * alpha + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
      m_run = m_new;
      alpha_pend = alpha;  // owed before block j's P.V, at the start of the next step
    } else {
      if (pend) {
        rescale(alpha_pend);
        accumulate(nxt, pbuf[nxt]);
      }
      alpha_pend = 1.0f;
      if (vis) {
        alpha_pend = fast ? softmax_fast(sacc, pbuf[cur])
                          : softmax_general(sacc, pbuf[cur], key0, diag, has_bias, cur);
        if (kStats && fast) count_fast(pbuf[cur]);
      }
      if (vis1) issue_s(nxt, sacc);
    }
    pend = vis;
    wait_loads();
    __syncthreads();
  };

  // prologue: K of the first two blocks and the first bias block; logits of the first block
  load_k(tile_of(0), 0);
  if (n_it > 1) load_k(tile_of(1), 1);
  load_b(tile_of(0), 0);
  wait_loads();
  __syncthreads();
  if (visible(tile_of(0))) issue_s(0, sacc);
  // step 0 reloads K buffer 0: every wave must have read block 0's K first
  __syncthreads();
  for (int it = 0; it < n_it; it += 2) {
    step(it, BufIndex<0>{});
    if (it + 1 < n_it) step(it + 1, BufIndex<1>{});
  }
  // the last block's P.V (its V landed before the last step's barrier)
  if (pend) {
    rescale(alpha_pend);
    if ((n_it - 1) & 1) accumulate(1, pbuf[1]);
    else accumulate(0, pbuf[0]);
  }

  // ---- epilogue: O = A / (S l) ----
  if (wave_active) {
    const float l_all = halves_sum(l_run);
    const float inv = 1.0f / (p.S * l_all);
    const int64_t row = ((int64_t)b * p.Hq + h) * p.N + myrow;
    if constexpr (!kDiag && !kMulti && kQ8 == 0) {
      // the log-sum-exp alone (no lost mass requested): the pipelined and the sequential
      // steps keep the same m and l bit for bit, so this equals the diagnostic kernel's
      if (g == 0 && p.lse && row_valid) p.lse[row] = (m_run + log2f(l_all)) * kLn2;
    }
    if constexpr (kDiag) {
      // log-sum-exp of the row's logits (natural units) and the lost non-sink mass fraction
      const float ns = halves_sum(l_ns), lo = halves_sum(l_lost);
      if (g == 0 && p.lse && row_valid) p.lse[row] = (m_run + log2f(l_all)) * kLn2;
      if (g == 0 && p.lost && row_valid) p.lost[row] = ns > 0.0f ? lo / ns : 0.0f;
    }
    float* orow = p.out + row * D;
    if (row_valid) {
#pragma unroll
      for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float4 v;
          v.x = oacc[dt][r4 * 4 + 0] * inv;
          v.y = oacc[dt][r4 * 4 + 1] * inv;
          v.z = oacc[dt][r4 * 4 + 2] * inv;
          v.w = oacc[dt][r4 * 4 + 3] * inv;
          *reinterpret_cast<float4*>(orow + dt * 32 + r4 * 8 + g * 4) = v;
        }
    }
  }
  if constexpr (kStats) {
    // fast blocks: every one of the lane's 32 pairs is visible and non-sink
    const unsigned int a = wave_sum(row_valid ? cnt_tot + 32u * n_fast : 0u),
                       z = wave_sum(row_valid ? cnt_zero + 32u * n_fast - (cnt_nz_fast >> 7) : 0u);
    if (lane == 0 && wave_active) {
      atomicAdd(&lds_cnt[wave / 2][0], a);
      atomicAdd(&lds_cnt[wave / 2][1], z);
    }
    __syncthreads();
    if (tid < 2 && (!kDiag || p.stats)) {
      const int r64 = row0 / kKvBlock + tid;  // 64-row block index
      if (r64 * kKvBlock < p.N) {
        unsigned long long* st = p.stats + 2 * (((int64_t)b * p.Hq + h) * n_tiles + r64);
        st[0] = lds_cnt[tid][0];
        st[1] = lds_cnt[tid][1];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode with split KV.  One wave per workgroup; workgroup (b, kv head, range)
// takes the G = Hq/Hkv query heads times Nq rows that read this kv head, packed
// into the 32 MFMA columns (lanes l and l + 32 hold packed row l: head l / Nq,
// query l % Nq; rows past G*Nq are padding with Q = 0), runs the P-cast pipeline
// over the range's key blocks from its own m = -inf, and writes the partial
// (m, l, A) and counters of each row.  pcast_decode_merge rescales the ranges to
// their common max and adds them.  Rows sit at the last Nq positions: row i sees
// keys j <= Nk - Nq + i.
// ---------------------------------------------------------------------------
template <int D, int kMode, bool kStats, bool kQ8>
__global__ __launch_bounds__(64) void pcast_decode_split(const Params p) {
  static_assert(kMode != kBf16, "FP8 modes only");
  using G = Geometry<D>;
  // kQ8: Q rounded here per row and K read as E4M3 codes with one scale per key block
  // (pcast_prepare_qk8's layout); the logits then run on the FP8 matrix cores
  constexpr int kKRow = kQ8 ? D : D * 2;
  constexpr int kSSteps = kQ8 ? D / 64 : G::kQSteps;  // logit MFMA k-steps per 32-key half
  using KFrag = typename Select<kQ8, i32x8_t, bf16x8_t>::type;
  constexpr int kVRow = kKvBlock;
  constexpr int kKTile = kKvBlock * kKRow;
  constexpr int kVTile = D * kVRow;
  using SK = Swizzle<kKRow>;
  using SV = Swizzle<kVRow>;
  constexpr int kKLoads = kKTile / 1024;  // 1 KB direct loads per block (one wave)
  constexpr int kVLoads = kVTile / 1024;
  // one K buffer, reloaded once the block's logits have read it; V and bias double
  // buffered (32.5 KiB: four workgroups per CU)
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[kKTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v0[kVTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v1[kVTile];
  __shared__ __attribute__((aligned(16))) float lds_b0[kKvBlock];
  __shared__ __attribute__((aligned(16))) float lds_b1[kKvBlock];
  auto vbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_v1 : lds_v0; };
  auto bbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_b1 : lds_b0; };

  const int lane = threadIdx.x;
  const int g = lane / 32, li = lane % 32;
  // key blocks of the cache; with Nk not a multiple of 64 the last one is partial
  const int n_blk = (p.Nk + kKvBlock - 1) / kKvBlock, n_full = p.Nk / kKvBlock;
  const int split = blockIdx.x % p.n_split;
  const int bhk = blockIdx.x / p.n_split;
  const int hk = bhk % p.Hkv, b = bhk / p.Hkv;
  const int Gq = p.Hq / p.Hkv;
  const bool row_ok = li < Gq * p.Nq;
  const int h = hk * Gq + (row_ok ? li / p.Nq : 0);
  const int qi = row_ok ? li % p.Nq : 0;
  const int pos = p.Nk - p.Nq + qi;  // the row's position
  const int t_first = split * p.split_blocks;
  const int t_end = min(t_first + p.split_blocks, n_blk);
  const int n_it = t_end - t_first;
  const bool with_bias = p.bias != nullptr;

  // Q operand as in the forward: bf16 Q[row][s*16 + g*8 .. +8), or the E4M3 codes of
  // Q[row][s*64 + g*32 .. +32) * 2^-e_row with the row's scale (padding rows are 0)
  KFrag qf[kSSteps];
  float c_row = p.logit_scale;  // log2(e)/sqrt(d), times 2^e_row with FP8 logits
  if constexpr (kQ8) {
    const uint16_t* qrow = p.q + (((int64_t)b * p.Hq + h) * p.Nq + qi) * D + g * 32;
    i32x4_t w[kSSteps][4];
    uint32_t m = 0;
#pragma unroll
    for (int s = 0; s < kSSteps; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const i32x4_t z = {};
        w[s][t] = row_ok ? *reinterpret_cast<const i32x4_t*>(qrow + s * 64 + t * 8) : z;
        m = max(m, absmax8(w[s][t]));
      }
    m = max(m, (uint32_t)__shfl_xor((int)m, 32));
    const int e = scale_exp(m);
#pragma unroll
    for (int s = 0; s < kSSteps; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        int lo, hi;
        codes8(w[s][t], e, lo, hi);
        qf[s][2 * t] = lo;
        qf[s][2 * t + 1] = hi;
      }
    c_row = ldexpf(p.logit_scale, e);
  } else {
    const uint16_t* qrow = p.q + (((int64_t)b * p.Hq + h) * p.Nq + qi) * D + g * 8;
#pragma unroll
    for (int s = 0; s < kSSteps; ++s) {
      bf16x8_t z = {};
      qf[s] = row_ok ? *reinterpret_cast<const bf16x8_t*>(qrow + s * 16) : z;
    }
  }
  // FP8 K codes are laid out in whole key blocks per head
  const uint8_t* kbase = kQ8 ? p.k8 + ((int64_t)b * p.Hkv + hk) * n_blk * kKTile
                             : reinterpret_cast<const uint8_t*>(p.k + ((int64_t)b * p.Hkv + hk) * p.Nk * D);
  const int* kexp_head = kQ8 ? p.kexp + ((int64_t)b * p.Hkv + hk) * n_blk : nullptr;
  const uint8_t* vbase = static_cast<const uint8_t*>(p.vop) + ((int64_t)b * p.Hkv + hk) * (int64_t)n_blk * kVTile;
  auto tile_of = [&](int it) __attribute__((always_inline)) { return p.order ? (t_end - 1 - it) : (t_first + it); };
  // load i fills LDS chunk position i * 64 + lane, which holds logical chunk position ^ key(row)
  auto load_k = [&](int t) __attribute__((always_inline)) {
    const uint8_t* ks = kbase + (int64_t)t * kKTile;
    // rows past Nk of a partial last block read row Nk - 1 instead (no row sees them)
    const int last = t < n_full ? kKvBlock - 1 : p.Nk - 1 - t * kKvBlock;
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int cp = i * 64 + lane, r = cp / SK::kChunks;
      load_to_lds16(ks + min(r, last) * kKRow + (((cp % SK::kChunks) ^ SK::key(r)) << 4), lds_k + i * 1024);
    }
  };
  auto load_v = [&](int t, int buf) __attribute__((always_inline)) {
    const uint8_t* vs = vbase + (int64_t)t * kVTile;
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      const int cp = i * 64 + lane, r = cp / SV::kChunks;
      load_to_lds16(vs + r * kVRow + (((cp % SV::kChunks) ^ SV::key(r)) << 4), vbuf(buf) + i * 1024);
    }
  };
  auto load_b = [&](int t, int buf) __attribute__((always_inline)) {
    if (with_bias) load_to_lds4(p.bias + min(t * kKvBlock + lane, p.Nk - 1), bbuf(buf));
  };
  auto wait_loads = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  const int xk = SK::key(li);
  auto issue_s = [&](f32x16_t(&sa)[2]) __attribute__((always_inline)) {
    const uint8_t* kl = lds_k + li * kKRow;
#pragma unroll
    for (int s = 0; s < kSSteps; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint8_t* kr = kl + kb * 32 * kKRow;
        if constexpr (kQ8) {
          const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(kr + (((4 * s + 2 * g) ^ xk) << 4));
          const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(kr + (((4 * s + 2 * g + 1) ^ xk) << 4));
          const i32x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          sa[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[s], s == 0 ? f32x16_t{} : sa[kb], 0, 0, 0, 0,
                                                                   0, 0);
        } else {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kr + (((2 * s + g) ^ xk) << 4));
          sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], s == 0 ? f32x16_t{} : sa[kb], 0, 0, 0);
        }
      }
  };
  f32x16_t oacc[G::kDTiles];
#pragma unroll
  for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
  auto accumulate = [&](int buf, const i32x8_t& pb) __attribute__((always_inline)) {
    const uint8_t* vl = vbuf(buf) + li * kVRow;
    const int xv = SV::key(li);
    const int vlo = ((2 * g) ^ xv) << 4, vhi = ((2 * g + 1) ^ xv) << 4;
#pragma unroll
    for (int dt = 0; dt < G::kDTiles; ++dt) {
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(vl + dt * 32 * kVRow + vlo);
      const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(vl + dt * 32 * kVRow + vhi);
      const i32x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, oacc[dt], 0, 0, 0, 0, 0, 0);
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  unsigned int cnt_tot = 0, cnt_zero = 0;
  f32x16_t sacc[2];
  i32x8_t pb;

  auto step = [&](int it, auto cur_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value, nxt = cur ^ 1;
    const int t = tile_of(it);
    // the logit scale of this block: times 2^e_block of K's scale with FP8 logits
    const float c = kQ8 ? ldexpf(c_row, kexp_head[t]) : c_row;
    if (it + 1 < n_it) {
      load_v(tile_of(it + 1), nxt);
      load_b(tile_of(it + 1), nxt);
    }
    issue_s(sacc);
    // the logits have read K (the MFMAs took their operands): reload it with block t+1
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (it + 1 < n_it) load_k(tile_of(it + 1));
    const int key0 = t * kKvBlock;
    const bool mask = key0 + kKvBlock - 1 > p.Nk - p.Nq;  // some row cannot see some key
    const bool has_bias = with_bias && __builtin_amdgcn_ballot_w64(bbuf(cur)[lane] != 0.0f) != 0;
    float bk[32];
    if (has_bias) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(bbuf(cur) + slot_key(g, 4 * q));
        bk[4 * q] = v.x; bk[4 * q + 1] = v.y; bk[4 * q + 2] = v.z; bk[4 * q + 3] = v.w;
      }
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float xj = has_bias ? fmaf(sacc[j / 16][j % 16], c, bk[j] * kLog2e) : sacc[j / 16][j % 16] * c;
      if (mask && key0 + slot_key(g, j) > pos) xj = -INFINITY;
      sacc[j / 16][j % 16] = xj;
    }
    float m4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m4[q] = fmaxf(sacc[q / 2][(q % 2) * 8], sacc[q / 2][(q % 2) * 8 + 1]);
#pragma unroll
      for (int r = 2; r < 8; r += 2)
        m4[q] = fmaxf(fmaxf(m4[q], sacc[q / 2][(q % 2) * 8 + r]), sacc[q / 2][(q % 2) * 8 + r + 1]);
    }
    // a row may see no key of a partial last block (Nk % 64 < Nq): then m_new stays -inf
    // while the row has seen nothing, and every p of the block is 0
    const float m_new = fmaxf(m_run, halves_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))));
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float pj = __builtin_amdgcn_exp2f(sacc[j / 16][j % 16] - m_use);
      sacc[j / 16][j % 16] = pj;
      ps[j % 4] += pj;
    }
    l_run = l_run * alpha + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
    m_run = m_new;
#pragma unroll
    for (int w = 0; w < 8; ++w)
      pb[w] = (int)cast4<kMode>(p, sacc[w / 4][4 * (w % 4)], sacc[w / 4][4 * (w % 4) + 1],
                                sacc[w / 4][4 * (w % 4) + 2], sacc[w / 4][4 * (w % 4) + 3]);
    if constexpr (kStats) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const bool vis = !mask || key0 + slot_key(g, j) <= pos;
        const bool nonsink = has_bias ? bk[j] == 0.0f : true;
        const bool z = (((uint32_t)pb[j / 4] >> (8 * (j % 4))) & 0xFFu) == 0;
        cnt_tot += (vis && nonsink);
        cnt_zero += (vis && nonsink && z);
      }
    }
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    accumulate(cur, pb);
    wait_loads();
    __syncthreads();
  };

  load_k(tile_of(0));
  load_v(tile_of(0), 0);
  load_b(tile_of(0), 0);
  wait_loads();
  __syncthreads();
  for (int it = 0; it < n_it; it += 2) {
    step(it, BufIndex<0>{});
    if (it + 1 < n_it) step(it + 1, BufIndex<1>{});
  }

  // partial results of this range, one slot per packed row
  const int64_t slot = ((int64_t)bhk * p.n_split + split) * 32 + li;
  float* arow = p.part_a + slot * D;
#pragma unroll
  for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 v;
      v.x = oacc[dt][r4 * 4 + 0];
      v.y = oacc[dt][r4 * 4 + 1];
      v.z = oacc[dt][r4 * 4 + 2];
      v.w = oacc[dt][r4 * 4 + 3];
      *reinterpret_cast<float4*>(arow + dt * 32 + r4 * 8 + g * 4) = v;
    }
  const float l_all = halves_sum(l_run);
  const unsigned int tot = cnt_tot + (unsigned int)__shfl_xor((int)cnt_tot, 32);
  const unsigned int zer = cnt_zero + (unsigned int)__shfl_xor((int)cnt_zero, 32);
  if (g == 0) {
    *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(m_run, l_all);
    if constexpr (kStats) {
      p.part_cnt[slot * 2] = row_ok ? tot : 0u;
      p.part_cnt[slot * 2 + 1] = row_ok ? zer : 0u;
    }
  }
}

// One workgroup per (b, kv head): thread t merges packed row t / 8, columns
// (t % 8) * 4 + 32 j, over the ranges: M = max m_r, O = sum 2^(m_r - M) A_r /
// (S sum 2^(m_r - M) l_r); counters are summed per (b, query head).
template <int D, bool kStats>
__global__ __launch_bounds__(256) void pcast_decode_merge(const Params p) {
  constexpr int kJ = D / 32;
  const int bhk = blockIdx.x;
  const int hk = bhk % p.Hkv, b = bhk / p.Hkv;
  const int Gq = p.Hq / p.Hkv;
  const int r = threadIdx.x / 8, cp = threadIdx.x % 8;
  const int R = Gq * p.Nq;
  __shared__ unsigned long long cnt[32][2];
  if (kStats && threadIdx.x < 64) cnt[threadIdx.x / 2][threadIdx.x % 2] = 0;
  __syncthreads();
  if (r < R) {
    const int64_t slot0 = (int64_t)bhk * p.n_split * 32 + r;
    float M = -INFINITY;
    for (int s = 0; s < p.n_split; ++s) M = fmaxf(M, p.part_ml[(slot0 + s * 32) * 2]);
    float L = 0.0f;
    float4 acc[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) acc[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    unsigned long long tot = 0, zer = 0;
    for (int s = 0; s < p.n_split; ++s) {
      const int64_t slot = slot0 + s * 32;
      const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + slot * 2);
      const float w = __builtin_amdgcn_exp2f(ml.x - M);
      L += w * ml.y;
      const float* a = p.part_a + slot * D + cp * 4;
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(a + j * 32);
        acc[j].x += w * v.x; acc[j].y += w * v.y; acc[j].z += w * v.z; acc[j].w += w * v.w;
      }
      if (kStats && cp == 0) {
        tot += p.part_cnt[slot * 2];
        zer += p.part_cnt[slot * 2 + 1];
      }
    }
    const float inv = 1.0f / (p.S * L);
    const int h = hk * Gq + r / p.Nq, qi = r % p.Nq;
    float* orow = p.out + (((int64_t)b * p.Hq + h) * p.Nq + qi) * D + cp * 4;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      *reinterpret_cast<float4*>(orow + j * 32) =
          make_float4(acc[j].x * inv, acc[j].y * inv, acc[j].z * inv, acc[j].w * inv);
    if (kStats && cp == 0) {
      atomicAdd(&cnt[r / p.Nq][0], tot);
      atomicAdd(&cnt[r / p.Nq][1], zer);
    }
  }
  if constexpr (kStats) {
    __syncthreads();
    if (threadIdx.x < Gq) {
      unsigned long long* st = p.stats + 2 * ((int64_t)b * p.Hq + hk * Gq + threadIdx.x);
      st[0] = cnt[threadIdx.x][0];
      st[1] = cnt[threadIdx.x][1];
    }
  }
}

// ---------------------------------------------------------------------------
// Backward by recomputation from the forward's log-sum-exp, the cast passed
// straight through: P = exp(s - lse), dP = dO V^T, dS = P (dP - D) with
// D = dO . O, dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d), dV = P^T dO.  All
// products on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS are
// rounded to bf16 for the products that take them as operands.
// ---------------------------------------------------------------------------

// Per row i: -D_i = -(dO_i . O_i), eight lanes per row, and -lse_i * sqrt(d), the
// log-sum-exp in the units of the raw logits q.k (both start the dK / dV kernel's
// accumulators, so that the products come out as dP - D and s - lse).
// Fill n 32-bit words with one value (the padded copies of the backward).
__global__ __launch_bounds__(256) void pcast_fill_u32(uint32_t* __restrict__ dst, uint32_t value, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = value;
}

template <int D>
__global__ __launch_bounds__(256) void pcast_bwd_rowdot(const uint16_t* __restrict__ dout, const float* __restrict__ o,
                                                        const float* __restrict__ lse, float* __restrict__ dvec,
                                                        float* __restrict__ nls, float sqrt_d, int64_t rows) {
  constexpr int kPer = D / 8;  // elements per lane
  const int64_t row = (int64_t)blockIdx.x * 32 + threadIdx.x / 8;
  const int part = threadIdx.x % 8;
  float acc = 0.0f;
  if (row < rows) {
    const uint16_t* a = dout + row * D + part * kPer;
    const float* b = o + row * D + part * kPer;
#pragma unroll
    for (int i = 0; i < kPer; i += 8) {
      const i32x4_t w = *reinterpret_cast<const i32x4_t*>(a + i);
      const float4 x = *reinterpret_cast<const float4*>(b + i);
      const float4 y = *reinterpret_cast<const float4*>(b + i + 4);
      acc = fmaf(__builtin_bit_cast(float, (uint32_t)w[0] << 16), x.x, acc);
      acc = fmaf(__builtin_bit_cast(float, (uint32_t)w[0] & 0xFFFF0000u), x.y, acc);
      acc = fmaf(__builtin_bit_cast(float, (uint32_t)w[1] << 16), x.z, acc);
      acc = fmaf(__builtin_bit_cast(float, (uint32_t)w[1] & 0xFFFF0000u), x.w, acc);
      acc = fmaf(__builtin_bit_cast(float, (uint32_t)w[2] << 16), y.x, acc);
      acc = fmaf(__builtin_bit_cast(float, (uint32_t)w[2] & 0xFFFF0000u), y.y, acc);
      acc = fmaf(__builtin_bit_cast(float, (uint32_t)w[3] << 16), y.z, acc);
      acc = fmaf(__builtin_bit_cast(float, (uint32_t)w[3] & 0xFFFF0000u), y.w, acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && part == 0) {
    dvec[row] = -acc;
    nls[row] = -lse[row] * sqrt_d;
  }
}

// dQ: a workgroup of 8 waves (two per SIMD) takes 256 query rows of one (b, h),
// a lane one row, and walks the key blocks: S^T = K Q^T and dP^T = V dO^T (keys x
// rows, the forward's layout), dS in registers, dQ^T += K^T dS^T with K^T read
// from the K tile by transposing LDS reads.  Each block is taken in its two 32-key
// halves (products, dS, then that half's k-steps of dQ), which keeps the wave
// within 256 registers.
constexpr int kDqWaves = 8;
constexpr int kDqRows = kDqWaves * kRowsPerWave;
template <int D, bool kCausal>
__global__ __launch_bounds__(kDqWaves * 64, 1) void pcast_attn_bwd_dq(const Params p) {
  using G = Geometry<D>;
  constexpr int kKRow = D * 2;
  constexpr int kKTile = kKvBlock * kKRow;
  using SK = SwizzleT<kKRow>;
  constexpr int kKLoads = kKTile / (1024 * kDqWaves);
  static_assert(kKTile % (1024 * kDqWaves) == 0, "staging split");
  __shared__ __attribute__((aligned(16))) uint8_t lds_k0[kKTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_k1[kKTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v0[kKTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v1[kKTile];
  __shared__ __attribute__((aligned(16))) float lds_b0[kKvBlock];
  __shared__ __attribute__((aligned(16))) float lds_b1[kKvBlock];
  auto kbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_k1 : lds_k0; };
  auto vbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_v1 : lds_v0; };
  auto bbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_b1 : lds_b0; };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int g = lane / 32, li = lane % 32;
  const int n_rb = (p.N + kDqRows - 1) / kDqRows;
  int b, h, rb;
  decode_block(blockIdx.x, n_rb * p.Hq * p.B, n_rb, p.Hq, kCausal, b, h, rb);
  const int hk = h / (p.Hq / p.Hkv);
  const int n_tiles = p.N / kKvBlock;
  const int row0 = rb * kDqRows;
  const int wrow0 = row0 + wave * kRowsPerWave;
  const int myrow = wrow0 + li;
  const bool wave_active = wrow0 < p.N;
  const int t_last = kCausal ? min((row0 + kDqRows - 1) / kKvBlock, n_tiles - 1) : n_tiles - 1;
  const int n_it = t_last + 1;
  const float c = p.logit_scale;
  const int64_t row = ((int64_t)b * p.Hq + h) * p.N + myrow;

  bf16x8_t qf[G::kQSteps], df[G::kQSteps];
  float lse2 = 0.0f, ndrow = 0.0f;
  if (wave_active) {
    const uint16_t* qrow = p.q + row * D + g * 8;
    const uint16_t* drw = p.dout + row * D + g * 8;
#pragma unroll
    for (int s = 0; s < G::kQSteps; ++s) {
      qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + s * 16);
      df[s] = *reinterpret_cast<const bf16x8_t*>(drw + s * 16);
    }
    lse2 = p.lse_in[row] * kLog2e;
    ndrow = p.dvec[row];
  }
  const __amdgpu_buffer_rsrc_t kres = buffer_rsrc(p.k + ((int64_t)b * p.Hkv + hk) * p.N * D);
  const __amdgpu_buffer_rsrc_t vres = buffer_rsrc(p.v + ((int64_t)b * p.Hkv + hk) * p.N * D);
  const __amdgpu_buffer_rsrc_t bres = buffer_rsrc(p.bias);
  int ksrc[kKLoads];
#pragma unroll
  for (int i = 0; i < kKLoads; ++i) {
    const int pos = (wave * kKLoads + i) * 64 + lane, r = pos / SK::kChunks;
    ksrc[i] = r * kKRow + (((pos % SK::kChunks) ^ SK::key(r)) << 4);
  }
  // Transposing reads of the K tile for the A operand of dQ^T += K^T dS^T: k-step s
  // of tile dt takes element e of lane (d row li, g) from key 16 s + 8 (e / 4) +
  // 4 g + e % 4, the slot order of dS; lane (group G, a) of a read addresses key
  // 16 s + 4 (G / 2) + a / 4 (+ 8 for elements 4..7) at column 32 dt + 16 (G % 2) +
  // 4 (a % 4).
  int tr_lo[G::kDTiles], tr_hi[G::kDTiles];
  {
    const int grp = lane / 16, a = lane % 16;
    const int r_lo = 4 * (grp / 2) + a / 4, r_hi = r_lo + 8;
#pragma unroll
    for (int dt = 0; dt < G::kDTiles; ++dt) {
      const int col = 32 * dt + 16 * (grp % 2) + 4 * (a % 4);
      tr_lo[dt] = r_lo * kKRow + ((((col >> 3) ^ SK::key(r_lo)) << 4) | ((col & 7) << 1));
      tr_hi[dt] = r_hi * kKRow + ((((col >> 3) ^ SK::key(r_hi)) << 4) | ((col & 7) << 1));
    }
  }
  const bool with_bias = p.bias != nullptr;
  auto visible = [&](int t) __attribute__((always_inline)) {
    return wave_active && (!kCausal || t * kKvBlock <= wrow0 + kRowsPerWave - 1);
  };
  auto load = [&](int t, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      buffer_to_lds16(kres, t * kKTile + ksrc[i], kbuf(buf) + (wave * kKLoads + i) * 1024);
      buffer_to_lds16(vres, t * kKTile + ksrc[i], vbuf(buf) + (wave * kKLoads + i) * 1024);
    }
    if (with_bias && wave == 0) buffer_to_lds4(bres, (t * kKvBlock + lane) * 4, bbuf(buf));
  };
  auto wait_loads = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  f32x16_t dqacc[G::kDTiles];
#pragma unroll
  for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[dt][r] = 0.0f;
  const int xk = SK::key(li);

  auto step = [&](int it, auto cur_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value, nxt = cur ^ 1;
    if (it + 1 < n_it) load(it + 1, nxt);
    if (visible(it)) {
      const int key0 = it * kKvBlock;
      const bool diag = kCausal && (key0 + kKvBlock - 1 > wrow0);
      const bool has_bias = with_bias && __builtin_amdgcn_ballot_w64(bbuf(cur)[lane] != 0.0f) != 0;
      const uint8_t* kl = kbuf(cur) + li * kKRow;
      const uint8_t* vl = vbuf(cur) + li * kKRow;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S^T and dP^T of the half's 32 keys
        f32x16_t sacc, pacc;
#pragma unroll
        for (int s = 0; s < G::kQSteps; ++s) {
          const int off = kb * 32 * kKRow + (((2 * s + g) ^ xk) << 4);
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kl + off);
          const bf16x8_t e = *reinterpret_cast<const bf16x8_t*>(vl + off);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], s == 0 ? f32x16_t{} : sacc, 0, 0, 0);
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e, df[s], s == 0 ? f32x16_t{} : pacc, 0, 0, 0);
        }
        uint32_t pw[8];
        if (!diag && !has_bias) {
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[2 * w], c, -lse2));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[2 * w + 1], c, -lse2));
            pw[w] = cast2_bf16(p0 * (pacc[2 * w] + ndrow), p1 * (pacc[2 * w + 1] + ndrow));
          }
        } else {
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            // the bias of the pair's two keys (adjacent slots)
            const float2 bk = has_bias ? *reinterpret_cast<const float2*>(bbuf(cur) + slot_key(g, 16 * kb + 2 * w))
                                       : float2{0.0f, 0.0f};
            float ds2[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int jj = 2 * w + e, j = 16 * kb + jj;
              const float bj = e ? bk.y : bk.x;
              const float x = has_bias ? fmaf(sacc[jj], c, bj * kLog2e) - lse2 : fmaf(sacc[jj], c, -lse2);
              float pj = __builtin_amdgcn_exp2f(x);
              if (diag && key0 + slot_key(g, j) > myrow) pj = 0.0f;
              ds2[e] = pj * (pacc[jj] + ndrow);
            }
            pw[w] = cast2_bf16(ds2[0], ds2[1]);
          }
        }
        // dQ^T += K^T dS^T over the half's two k-steps of 16 keys
#pragma unroll
        for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int s = 2 * kb + s2;
            const uint8_t* t = kbuf(cur) + s * 16 * kKRow;
            const bf16x8_t a = tr_frag(t + tr_lo[dt], t + tr_hi[dt]);
            const i32x4_t bw = {(int)pw[4 * s2], (int)pw[4 * s2 + 1], (int)pw[4 * s2 + 2], (int)pw[4 * s2 + 3]};
            dqacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bw), dqacc[dt], 0, 0, 0);
          }
      }
    }
    wait_loads();
    __syncthreads();
  };

  load(0, 0);
  wait_loads();
  __syncthreads();
  for (int it = 0; it < n_it; it += 2) {
    step(it, BufIndex<0>{});
    if (it + 1 < n_it) step(it + 1, BufIndex<1>{});
  }
  if (wave_active) {
    const float sc = p.logit_scale / kLog2e;  // 1 / sqrt(d)
    float* orow = p.dq + row * D;
#pragma unroll
    for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 v;
        v.x = dqacc[dt][r4 * 4 + 0] * sc;
        v.y = dqacc[dt][r4 * 4 + 1] * sc;
        v.z = dqacc[dt][r4 * 4 + 2] * sc;
        v.w = dqacc[dt][r4 * 4 + 3] * sc;
        *reinterpret_cast<float4*>(orow + dt * 32 + r4 * 8 + g * 4) = v;
      }
  }
}

// dK and dV: a workgroup of 4 waves takes 128 keys of one (b, kv head), a lane
// one key, and walks the 64-row query blocks of every query head that reads the
// kv head: S = Q K^T and dP = dO V^T (rows x keys: a lane holds its key's column),
// P and dS in registers, dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read
// from the dO and Q tiles by transposing LDS reads.
template <int D, bool kCausal>
__global__ __launch_bounds__(kThreads, 1) void pcast_attn_bwd_dkv(const Params p) {
  using G = Geometry<D>;
  constexpr int kRow = D * 2;
  constexpr int kTile = kKvBlock * kRow;
  using SR = SwizzleT<kRow>;
  constexpr int kLoads = kTile / (1024 * kWaves);
  static_assert(kTile % (1024 * kWaves) == 0, "staging split");
  __shared__ __attribute__((aligned(16))) uint8_t lds_q0[kTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_q1[kTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_o0[kTile];
  __shared__ __attribute__((aligned(16))) uint8_t lds_o1[kTile];
  __shared__ __attribute__((aligned(16))) float lds_l0[kKvBlock];
  __shared__ __attribute__((aligned(16))) float lds_l1[kKvBlock];
  __shared__ __attribute__((aligned(16))) float lds_d0[kKvBlock];
  __shared__ __attribute__((aligned(16))) float lds_d1[kKvBlock];
  auto qbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_q1 : lds_q0; };
  auto obuf = [&](int i) __attribute__((always_inline)) { return i ? lds_o1 : lds_o0; };
  auto lbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_l1 : lds_l0; };
  auto dbuf = [&](int i) __attribute__((always_inline)) { return i ? lds_d1 : lds_d0; };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int g = lane / 32, li = lane % 32;
  const int n_kb = (p.N + kBlockRows - 1) / kBlockRows;
  // the forward's XCD-aware order over (b, kv head, key block): the key blocks of a kv
  // head share one XCD's L2; ascending, so with a causal mask the key blocks with the
  // most rows start first
  int b, hk, kb;
  decode_block(blockIdx.x, n_kb * p.Hkv * p.B, n_kb, p.Hkv, false, b, hk, kb);
  const int Gq = p.Hq / p.Hkv;
  const int key0 = kb * kBlockRows;
  const int wkey0 = key0 + wave * kRowsPerWave;
  const int mykey = wkey0 + li;
  const bool wave_active = wkey0 < p.N;
  const int n_rblk = p.N / kKvBlock;
  const int r_first = kCausal ? key0 / kKvBlock : 0;
  const int n_r = n_rblk - r_first;
  const int n_it = Gq * n_r;
  const float c = p.logit_scale;
  const int64_t krow = ((int64_t)b * p.Hkv + hk) * p.N + mykey;

  bf16x8_t kf[G::kQSteps], vf[G::kQSteps];
  float bkl = 0.0f;
  if (wave_active) {
    const uint16_t* kr = p.k + krow * D + g * 8;
    const uint16_t* vr = p.v + krow * D + g * 8;
#pragma unroll
    for (int s = 0; s < G::kQSteps; ++s) {
      kf[s] = *reinterpret_cast<const bf16x8_t*>(kr + s * 16);
      vf[s] = *reinterpret_cast<const bf16x8_t*>(vr + s * 16);
    }
    if (p.bias) bkl = p.bias[mykey] * kLog2e;
  }
  int rsrc[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int pos = (wave * kLoads + i) * 64 + lane, r = pos / SR::kChunks;
    rsrc[i] = r * kRow + (((pos % SR::kChunks) ^ SR::key(r)) << 4);
  }
  // Transposing reads of the Q and dO tiles for the A operands of dV^T += dO^T P and
  // dK^T += Q^T dS: k-step st of tile dt takes element e of lane (d row li, g) from
  // query row 16 st + 8 (e / 4) + 4 g + e % 4, the slot order of P and dS.  Lane
  // (group G, a) of a read addresses row 16 st + 4 (G / 2) + a / 4 (+ 8 for elements
  // 4..7) at column 32 dt + 16 (G % 2) + 4 (a % 4); the row's swizzle key does not
  // depend on st.
  int tr_lo[G::kDTiles], tr_hi[G::kDTiles];
  {
    const int grp = lane / 16, a = lane % 16;
    const int r_lo = 4 * (grp / 2) + a / 4, r_hi = r_lo + 8;
#pragma unroll
    for (int dt = 0; dt < G::kDTiles; ++dt) {
      const int col = 32 * dt + 16 * (grp % 2) + 4 * (a % 4);
      tr_lo[dt] = r_lo * kRow + ((((col >> 3) ^ SR::key(r_lo)) << 4) | ((col & 7) << 1));
      tr_hi[dt] = r_hi * kRow + ((((col >> 3) ^ SR::key(r_hi)) << 4) | ((col & 7) << 1));
    }
  }
  // iteration it: query head hk * Gq + it / n_r, row blocks from the last one down, so
  // that the workgroups of a kv head, whatever their first row block, read the same
  // Q / dO tiles at about the same time
  auto head_of = [&](int it) __attribute__((always_inline)) { return hk * Gq + it / n_r; };
  auto rblk_of = [&](int it) __attribute__((always_inline)) { return n_rblk - 1 - it % n_r; };
  auto load = [&](int it, int buf) __attribute__((always_inline)) {
    const int64_t hrow = ((int64_t)b * p.Hq + head_of(it)) * p.N;  // first row of the head
    const int r = rblk_of(it);
    const __amdgpu_buffer_rsrc_t qs = buffer_rsrc(p.q + hrow * D), os = buffer_rsrc(p.dout + hrow * D);
    const int toff = r * kTile;  // the block's byte offset within the head
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      buffer_to_lds16(qs, toff + rsrc[i], qbuf(buf) + (wave * kLoads + i) * 1024);
      buffer_to_lds16(os, toff + rsrc[i], obuf(buf) + (wave * kLoads + i) * 1024);
    }
    if (wave == 0) {
      buffer_to_lds4(buffer_rsrc(p.nls + hrow), (r * kKvBlock + lane) * 4, lbuf(buf));
      buffer_to_lds4(buffer_rsrc(p.dvec + hrow), (r * kKvBlock + lane) * 4, dbuf(buf));
    }
  };
  auto wait_loads = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  f32x16_t dkacc[G::kDTiles], dvacc[G::kDTiles];
#pragma unroll
  for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkacc[dt][r] = 0.0f;
      dvacc[dt][r] = 0.0f;
    }
  const int xr = SR::key(li);
  // One block of 64 query rows, in two 32-row halves hh: the S and dP products of
  // half 0, then of half 1 while half 0's P and dS are formed, then half 0's dV and
  // dK k-steps while half 1's are formed, then half 1's.  Each MFMA sits in a chunk
  // of its own with the operand fragment of the MFMA kAhead later and a slice of
  // the VALU work; sched_barrier fences keep the chunks in order.  The S
  // accumulator of a half starts at -lse * sqrt(d) of its rows (-inf where the
  // causal mask hides the pair) and the dP accumulator at -D, so the products
  // come out as s - lse and dP - D and a pair costs one fma, one exp2, one
  // multiply and a conversion.
  auto block = [&](auto cur_c, bool diag, int rrow0) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr int kA = 2 * G::kQSteps;   // S and dP MFMAs of one half
    constexpr int kC = 4 * G::kDTiles;   // dV and dK MFMAs of one half (two k-steps)
    constexpr int kM = 2 * kA + 2 * kC;  // the block's MFMAs
    constexpr int kAhead = 3, kRing = kAhead + 1;
    const uint8_t* ql = qbuf(cur) + li * kRow;
    const uint8_t* ol = obuf(cur) + li * kRow;
    const int lim = mykey - rrow0 - 4 * g;
    f32x16_t sacc[2], pacc[2];
    uint32_t pp[2][8], ps[2][8];
    bf16x8_t ring[kRing];
    // accumulator starts: element e of half hh is row 32 hh + 8 (e / 4) + 4 g + e % 4
    // of the block (slot order), whose -lse sqrt(d) and -D sit in the staged rows
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a = *reinterpret_cast<const float4*>(lbuf(cur) + 32 * hh + 8 * q + 4 * g);
        const float4 e = *reinterpret_cast<const float4*>(dbuf(cur) + 32 * hh + 8 * q + 4 * g);
        sacc[hh][4 * q] = a.x; sacc[hh][4 * q + 1] = a.y; sacc[hh][4 * q + 2] = a.z; sacc[hh][4 * q + 3] = a.w;
        pacc[hh][4 * q] = e.x; pacc[hh][4 * q + 1] = e.y; pacc[hh][4 * q + 2] = e.z; pacc[hh][4 * q + 3] = e.w;
      }
    if (kCausal && diag) {
      // row rrow0 + slot_key(g, j) is masked when it lies above the key: slot_key(0, j) <
      // lim with lim = mykey - rrow0 - 4 g
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (slot_key(0, 16 * hh + e) < lim) sacc[hh][e] = -INFINITY;
    }
    // MFMA i: i < 2 kA: half i / kA, k-step (i % kA) / 2, S (even) or dP (odd);
    // then half hh = (i - 2 kA) / kC and q = (i - 2 kA) % kC: k-step 2 hh + q / (2 kDTiles),
    // tile (q / 2) % kDTiles, dV (even) or dK (odd)
    auto fetch = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < 2 * kA) {
        constexpr int hh = i / kA, r = i % kA, st = r / 2;
        const int off = hh * 32 * kRow + (((2 * st + g) ^ xr) << 4);
        ring[i % kRing] = *reinterpret_cast<const bf16x8_t*>((r % 2 ? ol : ql) + off);
      } else if constexpr (i < kM) {
        constexpr int r = i - 2 * kA, hh = r / kC, q = r % kC, dt = (q / 2) % G::kDTiles;
        constexpr int st = 2 * hh + q / (2 * G::kDTiles);
        const uint8_t* t = (q % 2 ? qbuf(cur) : obuf(cur)) + st * 16 * kRow;
        ring[i % kRing] = tr_frag(t + tr_lo[dt], t + tr_hi[dt]);
      }
    };
    auto mfma = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      const bf16x8_t& a = ring[i % kRing];
      if constexpr (i < 2 * kA) {
        constexpr int hh = i / kA, r = i % kA, st = r / 2;
        if constexpr (r % 2 == 0)
          sacc[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[st], sacc[hh], 0, 0, 0);
        else
          pacc[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[st], pacc[hh], 0, 0, 0);
      } else {
        constexpr int r = i - 2 * kA, hh = r / kC, q = r % kC, s2 = q / (2 * G::kDTiles), dt = (q / 2) % G::kDTiles;
        const uint32_t* src = q % 2 == 0 ? pp[hh] : ps[hh];
        const i32x4_t bw = {(int)src[4 * s2], (int)src[4 * s2 + 1], (int)src[4 * s2 + 2], (int)src[4 * s2 + 3]};
        if constexpr (q % 2 == 0)
          dvacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bw), dvacc[dt], 0, 0, 0);
        else
          dkacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bw), dkacc[dt], 0, 0, 0);
      }
    };
    auto unit = [&](auto nc) __attribute__((always_inline)) {  // P and dS of rows 2w, 2w + 1
      constexpr int n = decltype(nc)::value, hh = n / 8, w = n % 8;
      const float pj0 = __builtin_amdgcn_exp2f(fmaf(sacc[hh][2 * w], c, bkl));
      const float pj1 = __builtin_amdgcn_exp2f(fmaf(sacc[hh][2 * w + 1], c, bkl));
      pp[hh][w] = cast2_bf16(pj0, pj1);
      ps[hh][w] = cast2_bf16(pj0 * pacc[hh][2 * w], pj1 * pacc[hh][2 * w + 1]);
    };
#define PCAST_FENCE __builtin_amdgcn_sched_barrier(0)
    static_for<kAhead>([&](auto ic) __attribute__((always_inline)) { fetch(ic); });
    PCAST_FENCE;
    static_for<kM>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      mfma(ic);
      fetch(IC<i + kAhead>{});
      // half 0's units over the S / dP MFMAs of half 1, half 1's over the dV / dK
      // MFMAs of half 0
      if constexpr (i >= kA && i < 2 * kA) {
        constexpr int c0 = i - kA, u0 = c0 * 8 / kA, u1 = (c0 + 1) * 8 / kA;
        static_for<u1 - u0>([&](auto uc) __attribute__((always_inline)) { unit(IC<u0 + decltype(uc)::value>{}); });
      } else if constexpr (i >= 2 * kA && i < 2 * kA + kC) {
        constexpr int c0 = i - 2 * kA, u0 = c0 * 8 / kC, u1 = (c0 + 1) * 8 / kC;
        static_for<u1 - u0>([&](auto uc) __attribute__((always_inline)) { unit(IC<8 + u0 + decltype(uc)::value>{}); });
      }
      PCAST_FENCE;
    });
#undef PCAST_FENCE
  };

  auto step = [&](int it, auto cur_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value, nxt = cur ^ 1;
    if (it + 1 < n_it) load(it + 1, nxt);
    const int rrow0 = rblk_of(it) * kKvBlock;
    // one code path for masked and unmasked blocks, the mask only in the accumulator
    // starts (with two paths the register allocator moves the dK / dV accumulators
    // between register files where they join)
    if (wave_active && (!kCausal || rrow0 + kKvBlock - 1 >= wkey0))
      block(cur_c, rrow0 < wkey0 + kRowsPerWave - 1, rrow0);
    wait_loads();
    __syncthreads();
  };

  load(0, 0);
  wait_loads();
  __syncthreads();
  for (int it = 0; it < n_it; it += 2) {
    step(it, BufIndex<0>{});
    if (it + 1 < n_it) step(it + 1, BufIndex<1>{});
  }
  if (wave_active) {
    const float sc = p.logit_scale / kLog2e;  // 1 / sqrt(d)
    float* krw = p.dk + krow * D;
    float* vrw = p.dv + krow * D;
#pragma unroll
    for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 a, e;
        a.x = dkacc[dt][r4 * 4 + 0] * sc; a.y = dkacc[dt][r4 * 4 + 1] * sc;
        a.z = dkacc[dt][r4 * 4 + 2] * sc; a.w = dkacc[dt][r4 * 4 + 3] * sc;
        e.x = dvacc[dt][r4 * 4 + 0]; e.y = dvacc[dt][r4 * 4 + 1];
        e.z = dvacc[dt][r4 * 4 + 2]; e.w = dvacc[dt][r4 * 4 + 3];
        *reinterpret_cast<float4*>(krw + dt * 32 + r4 * 8 + g * 4) = a;
        *reinterpret_cast<float4*>(vrw + dt * 32 + r4 * 8 + g * 4) = e;
      }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PCAST_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// 0: gfx950, 1: other arch, -1: unknown.  Cached per device.
int arch_check(int dev) {
  static std::mutex mu;
  static int cache[64];
  static bool init = false;
  std::lock_guard<std::mutex> lock(mu);
  if (!init) {
    for (int& c : cache) c = -1;
    init = true;
  }
  if (dev < 0 || dev >= 64) return 1;
  if (cache[dev] < 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
    cache[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 0 : 1;
  }
  return cache[dev];
}

// Device address of `scratch` on the current device, looked up once per device.
int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(PCAST_ENOTSUP, "device %d: at most 64 devices", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(PCAST_EHIP, "hipGetSymbolAddress(scratch) returned null");
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return PCAST_OK;
}

bool is_pow2(float S) {
  int e;
  return std::frexp(S, &e) == 0.5f;
}

template <int D, bool kFp8>
void launch_prep(const uint16_t* V, void* ws, int64_t n_blocks, int N, hipStream_t stream) {
  const int n_tiles = (N + kKvBlock - 1) / kKvBlock;
  hipLaunchKernelGGL((pcast_prep_v<D, kFp8>), dim3((unsigned)n_blocks), dim3(256), 0, stream, V, ws, N, n_tiles);
}

template <int D, int kMode, bool kCausal>
void launch_attn3(const Params& p, hipStream_t stream) {
  const int n_rb = (p.N + kBlockRows - 1) / kBlockRows;
  const dim3 grid((unsigned)(n_rb * p.Hq * p.B));
  if constexpr (kMode == kBf16) {
    if (p.stats)
      hipLaunchKernelGGL((pcast_attn_fwd_bf16<D, kCausal, true>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((pcast_attn_fwd_bf16<D, kCausal, false>), grid, dim3(kThreads), 0, stream, p);
  } else if (p.k8 && p.q8) {
    if (p.stats)
      hipLaunchKernelGGL((pcast_attn_fwd_fp8<D, kMode, kCausal, 1, 2>), grid, dim3(kThreads), 0, stream, p, NoCells{});
    else
      hipLaunchKernelGGL((pcast_attn_fwd_fp8<D, kMode, kCausal, 0, 2>), grid, dim3(kThreads), 0, stream, p, NoCells{});
  } else if (p.k8) {
    if (p.stats)
      hipLaunchKernelGGL((pcast_attn_fwd_fp8<D, kMode, kCausal, 1, 1>), grid, dim3(kThreads), 0, stream, p, NoCells{});
    else
      hipLaunchKernelGGL((pcast_attn_fwd_fp8<D, kMode, kCausal, 0, 1>), grid, dim3(kThreads), 0, stream, p, NoCells{});
  } else if (p.lost) {
    // the lost mass needs the per-key work of the sequential step in every block; the
    // log-sum-exp alone is written by the pipelined kernels below
    hipLaunchKernelGGL((pcast_attn_fwd_fp8<D, kMode, kCausal, 2, 0>), grid, dim3(kThreads), 0, stream, p, NoCells{});
  } else {
    if (p.stats)
      hipLaunchKernelGGL((pcast_attn_fwd_fp8<D, kMode, kCausal, 1, 0>), grid, dim3(kThreads), 0, stream, p, NoCells{});
    else
      hipLaunchKernelGGL((pcast_attn_fwd_fp8<D, kMode, kCausal, 0, 0>), grid, dim3(kThreads), 0, stream, p, NoCells{});
  }
}

template <int D, int kMode>
void launch_attn2(const Params& p, int causal, hipStream_t stream) {
  if (causal) launch_attn3<D, kMode, true>(p, stream);
  else launch_attn3<D, kMode, false>(p, stream);
}

template <int D>
void launch_attn(const Params& p, int mode, int causal, hipStream_t stream) {
  switch (mode) {
    case kPow2: launch_attn2<D, kPow2>(p, causal, stream); break;
    case kPow2Clamp: launch_attn2<D, kPow2Clamp>(p, causal, stream); break;
    case kMul: launch_attn2<D, kMul>(p, causal, stream); break;
    case kMulClamp: launch_attn2<D, kMulClamp>(p, causal, stream); break;
    default: launch_attn2<D, kBf16>(p, causal, stream); break;
  }
}

template <int D, int kMode, bool kCausal>
void launch_multi3(const Params& p, const Cells& cells, bool stats, hipStream_t stream) {
  const int n_rb = (p.N + kBlockRows - 1) / kBlockRows;
  const dim3 grid((unsigned)(n_rb * p.Hq * p.B * cells.n));
  if (stats)
    hipLaunchKernelGGL((pcast_attn_fwd_fp8<D, kMode, kCausal, 1, 0, true>), grid, dim3(kThreads), 0, stream, p, cells);
  else
    hipLaunchKernelGGL((pcast_attn_fwd_fp8<D, kMode, kCausal, 0, 0, true>), grid, dim3(kThreads), 0, stream, p, cells);
}

template <int D, int kMode>
void launch_multi2(const Params& p, const Cells& cells, int causal, bool stats, hipStream_t stream) {
  if (causal) launch_multi3<D, kMode, true>(p, cells, stats, stream);
  else launch_multi3<D, kMode, false>(p, cells, stats, stream);
}

template <int D>
void launch_multi(const Params& p, const Cells& cells, int mode, int causal, bool stats, hipStream_t stream) {
  switch (mode) {
    case kPow2: launch_multi2<D, kPow2>(p, cells, causal, stats, stream); break;
    case kPow2Clamp: launch_multi2<D, kPow2Clamp>(p, cells, causal, stats, stream); break;
    case kMul: launch_multi2<D, kMul>(p, cells, causal, stats, stream); break;
    default: launch_multi2<D, kMulClamp>(p, cells, causal, stats, stream); break;
  }
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// Workspace of the backward: per row, -D = -(dO . O), then -lse * sqrt(d) (fp32,
// [B][Hq][N] each); 256-aligned parts.
struct BwdLayout {
  size_t dvec, nls, total;
};
BwdLayout bwd_layout(int B, int Hq, int /*Hkv*/, int N, int /*d*/) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  BwdLayout l;
  l.dvec = 0;
  l.nls = up((size_t)B * Hq * N * 4);
  l.total = l.nls + up((size_t)B * Hq * N * 4);
  return l;
}

// With N not a multiple of 64 the backward runs on copies padded to Np = whole key blocks:
// Q, K, V, dO (bf16) and O (fp32) with zero rows past N, lse with zeros, a bias of 0
// (or the caller's) on the first N keys and -inf past them, and the three gradients; the
// padded rows and keys contribute exactly nothing (their P is 0, or their dO is 0), and
// the gradients of the first N rows are copied back.  Offsets after the row workspace of
// Np, 256-aligned each.
struct BwdPad {
  int Np;
  size_t q, k, v, o, dout, lse, bias, dq, dk, dv, total;
};
BwdPad bwd_pad_layout(int B, int Hq, int Hkv, int N, int d) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  BwdPad l;
  l.Np = (N + kKvBlock - 1) / kKvBlock * kKvBlock;
  const size_t nq = (size_t)B * Hq * l.Np * d, nk = (size_t)B * Hkv * l.Np * d;
  l.q = up(bwd_layout(B, Hq, Hkv, l.Np, d).total);
  l.k = up(l.q + nq * 2);
  l.v = up(l.k + nk * 2);
  l.o = up(l.v + nk * 2);
  l.dout = up(l.o + nq * 4);
  l.lse = up(l.dout + nq * 2);
  l.bias = up(l.lse + (size_t)B * Hq * l.Np * 4);
  l.dq = up(l.bias + (size_t)l.Np * 4);
  l.dk = up(l.dq + nq * 4);
  l.dv = up(l.dk + nk * 4);
  l.total = up(l.dv + nk * 4);
  return l;
}

// Workspace of the split-KV decode: per (b, kv head, range, packed row) the partial
// accumulator [D] fp32, then (m, l) fp32, then the two counters u32; 256-aligned parts.
struct DecodeLayout {
  int n_split;
  size_t a, ml, cnt, total;
};
DecodeLayout decode_layout(int B, int Hkv, int Nk, int d, int split_keys) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  DecodeLayout l;
  l.n_split = (Nk + split_keys - 1) / split_keys;
  const size_t slots = (size_t)B * Hkv * l.n_split * 32;
  l.a = 0;
  l.ml = up(slots * d * 4);
  l.cnt = up(l.ml + slots * 2 * 4);
  l.total = up(l.cnt + slots * 2 * 4);
  return l;
}

// Workspace of the FP8-logit path, byte offsets from its start (each 256-aligned):
// the V operand copy (as in the plain workspace), the E4M3 codes of K in K's own
// layout, and the exponent of each key block's scale (int32).
struct Qk8Layout {
  size_t k8, kexp, total;
  size_t q8, qexp, total_rot;  // the rotated variant adds the codes and row exponents of Q
};
Qk8Layout qk8_layout(int B, int Hkv, int N, int d, int Hq = 0) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t n_tiles = (size_t)(N + kKvBlock - 1) / kKvBlock;
  const size_t nkv = (size_t)B * Hkv * n_tiles * kKvBlock * d;  // whole key blocks
  Qk8Layout l;
  l.k8 = up(nkv);
  l.kexp = up(l.k8 + nkv);
  l.total = up(l.kexp + (size_t)B * Hkv * n_tiles * 4);
  l.q8 = l.total;
  l.qexp = up(l.q8 + (size_t)B * Hq * N * d);
  l.total_rot = up(l.qexp + (size_t)B * Hq * N * 4);
  return l;
}

}  // namespace

extern "C" {

size_t pcast_stats_words(int B, int Hq, int N) {
  if (B <= 0 || Hq <= 0 || N <= 0) return 0;
  return (size_t)B * Hq * ((N + kKvBlock - 1) / kKvBlock) * 2;
}

size_t pcast_workspace_bytes(int B, int Hkv, int N, int d, float S) {
  if (B <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return 0;
  const size_t keys = (size_t)(N + kKvBlock - 1) / kKvBlock * kKvBlock;  // whole key blocks
  return (size_t)B * Hkv * keys * d * ((S == 0.0f) ? 2 : 1);
}

size_t pcast_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return 0;
  return N % kKvBlock ? bwd_pad_layout(B, Hq, Hkv, N, d).total : bwd_layout(B, Hq, Hkv, N, d).total;
}

size_t pcast_decode_workspace_bytes(int B, int Hkv, int Nk, int d, int split_keys) {
  if (B <= 0 || Hkv <= 0 || Nk <= 0 || d <= 0 || split_keys <= 0) return 0;
  return decode_layout(B, Hkv, Nk, d, split_keys).total;
}

size_t pcast_workspace_bytes_qk8_rot(int B, int Hq, int Hkv, int N, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return 0;
  return qk8_layout(B, Hkv, N, d, Hq).total_rot;
}

size_t pcast_workspace_bytes_qk8(int B, int Hkv, int N, int d) {
  if (B <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return 0;
  return qk8_layout(B, Hkv, N, d).total;
}

int pcast_abi_version(void) { return PCAST_ABI_VERSION; }

const char* pcast_strerror(int code) {
  static thread_local char buf[640];
  const char* base = code == PCAST_OK       ? "success"
                     : code == PCAST_EINVAL  ? "invalid argument"
                     : code == PCAST_ENOTSUP ? "not supported"
                     : code == PCAST_EHIP    ? "HIP runtime error"
                                             : "unknown error code";
  if (code != PCAST_OK && g_last_error[0])
    std::snprintf(buf, sizeof(buf), "%s: %s", base, g_last_error);
  else
    std::snprintf(buf, sizeof(buf), "%s", base);
  return buf;
}

}  // extern "C"

namespace {

// Shape and scalar checks shared by the entry points.  Nothing here touches the device.
// any_n: the entry point takes any N >= 1, a partial last key block being masked past
// N; otherwise N must be a multiple of 64.
int check_shape(int B, int Hq, int Hkv, int N, int d, float S, bool any_n = false) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0)
    return fail(PCAST_EINVAL, "B, Hq, Hkv, N, d must be positive");
  if (Hq % Hkv != 0) return fail(PCAST_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (!std::isfinite(S) || S < 0.0f) return fail(PCAST_EINVAL, "S must be finite and >= 0");
  if (d != 64 && d != 128) return fail(PCAST_ENOTSUP, "d = %d: supported head sizes are 64 and 128", d);
  if (N % kKvBlock != 0 && !any_n)
    return fail(PCAST_ENOTSUP, "N = %d: must be a multiple of %d for this entry point", N, kKvBlock);
  if ((int64_t)B * Hkv * ((N + kKvBlock - 1) / kKvBlock) > (int64_t)INT32_MAX ||
      (int64_t)B * Hq * ((N + kBlockRows - 1) / kBlockRows) > (int64_t)INT32_MAX)
    return fail(PCAST_ENOTSUP, "grid too large");
  return PCAST_OK;
}

int check_attn_args(const void* Q, const void* K, const float* bias, int causal, int order,
                    const float* out, const unsigned long long* stats) {
  if (!Q || !K || !out) return fail(PCAST_EINVAL, "Q, K and out must be non-null");
  if (causal != 0 && causal != 1) return fail(PCAST_EINVAL, "causal must be 0 or 1");
  if (order != PCAST_ORDER_FORWARD && order != PCAST_ORDER_REVERSE)
    return fail(PCAST_EINVAL, "order must be 0 (forward) or 1 (reverse)");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(out, 16))
    return fail(PCAST_EINVAL, "Q, K and out must be 16-byte aligned");
  if (bias && !aligned(bias, 4)) return fail(PCAST_EINVAL, "bias must be 4-byte aligned");
  if (stats && !aligned(stats, 8)) return fail(PCAST_EINVAL, "stats must be 8-byte aligned");
  return PCAST_OK;
}

int check_device() {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  const int arch = arch_check(dev);
  if (arch < 0) return fail(PCAST_EHIP, "cannot query device %d", dev);
  if (arch > 0) return fail(PCAST_ENOTSUP, "device %d is not gfx950", dev);
  return PCAST_OK;
}

int enqueue_prep(const void* V, int B, int Hkv, int N, int d, float S, void* ws, hipStream_t st) {
  const bool fp8 = S != 0.0f;
  const int64_t n_blocks = (int64_t)B * Hkv * ((N + kKvBlock - 1) / kKvBlock);
  const uint16_t* Vb = static_cast<const uint16_t*>(V);
  if (d == 64) {
    if (fp8) launch_prep<64, true>(Vb, ws, n_blocks, N, st); else launch_prep<64, false>(Vb, ws, n_blocks, N, st);
  } else {
    if (fp8) launch_prep<128, true>(Vb, ws, n_blocks, N, st); else launch_prep<128, false>(Vb, ws, n_blocks, N, st);
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PCAST_OK : hip_fail(e, "V pre-pass launch");
}

// K codes and block exponents, and the FP8 V operand copy, in one pass over the key blocks.
int enqueue_prep_qk8(const void* K, const void* V, int B, int Hkv, int N, int d, void* ws, hipStream_t st) {
  const Qk8Layout l = qk8_layout(B, Hkv, N, d);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const int n_tiles = (N + kKvBlock - 1) / kKvBlock;
  const int64_t n_blocks = (int64_t)B * Hkv * n_tiles;
  const uint16_t* Kb = static_cast<const uint16_t*>(K);
  const uint16_t* Vb = static_cast<const uint16_t*>(V);
  int* kexp = reinterpret_cast<int*>(base + l.kexp);
  if (d == 64)
    hipLaunchKernelGGL(pcast_prep_kv8<64>, dim3((unsigned)n_blocks), dim3(256), 0, st, Kb, Vb, base, base + l.k8, kexp,
                       N, n_tiles);
  else
    hipLaunchKernelGGL(pcast_prep_kv8<128>, dim3((unsigned)n_blocks), dim3(256), 0, st, Kb, Vb, base, base + l.k8,
                       kexp, N, n_tiles);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PCAST_OK : hip_fail(e, "K/V pre-pass launch");
}

// The FP8-logit path needs the FP8 P.V path.
int check_qk8(float S) {
  if (S == 0.0f) return fail(PCAST_ENOTSUP, "FP8 logits need S > 0 (the FP8 P.V path)");
  return PCAST_OK;
}

int enqueue_attn(const void* Q, const void* K, const void* ws, const float* bias, int B, int Hq,
                 int Hkv, int N, int d, int causal, float S, int order, float* out,
                 unsigned long long* stats, hipStream_t st, bool qk8 = false, float* lse = nullptr,
                 float* lost = nullptr, bool rot = false) {
  const bool fp8 = S != 0.0f;
  Params p{};
  p.lse = lse;
  p.lost = lost;
  if (qk8) {
    const Qk8Layout l = qk8_layout(B, Hkv, N, d, Hq);
    const uint8_t* base = static_cast<const uint8_t*>(ws);
    p.k8 = base + l.k8;
    p.kexp = reinterpret_cast<const int*>(base + l.kexp);
    if (rot) {
      p.q8 = base + l.q8;
      p.qexp = reinterpret_cast<const int*>(base + l.qexp);
    }
  }
  p.q = static_cast<const uint16_t*>(Q);
  p.k = static_cast<const uint16_t*>(K);
  p.vop = ws;
  p.bias = bias;
  p.out = out;
  p.stats = stats;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N;
  p.order = order;
  p.logit_scale = (float)(1.4426950408889634 / std::sqrt((double)d));
  p.S = fp8 ? S : 1.0f;
  p.inv_S = fp8 ? 1.0f / S : 1.0f;
  // S > 448: P is clamped to 448/S so that S*P stays at or below 448 (exact for S = 2^k;
  // otherwise S*fl(448/S) may exceed 448 by an ulp, which still rounds to 448).
  p.p_clamp = fp8 ? 448.0f / S : 1.0f;
  const int mode = !fp8 ? kBf16 : ((is_pow2(S) ? kPow2 : kMul) + (S > 448.0f ? 1 : 0));
  if (d == 64) launch_attn<64>(p, mode, causal, st);
  else launch_attn<128>(p, mode, causal, st);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PCAST_OK : hip_fail(e, "attention kernel launch");
}

// Argument checks shared by the decode entry points (Q, out, workspace; shapes).
int check_decode(const void* Q, const float* bias, int B, int Hq, int Hkv, int Nq, int Nk, int d, float S,
                 int order, int split_keys, const float* out, const unsigned long long* stats,
                 const void* workspace, bool any_nk) {
  if (!aligned(Q, 16) || !aligned(out, 16) || !aligned(workspace, 16))
    return fail(PCAST_EINVAL, "Q, out and workspace must be 16-byte aligned");
  if (bias && !aligned(bias, 4)) return fail(PCAST_EINVAL, "bias must be 4-byte aligned");
  if (stats && !aligned(stats, 8)) return fail(PCAST_EINVAL, "stats must be 8-byte aligned");
  if (order != PCAST_ORDER_FORWARD && order != PCAST_ORDER_REVERSE)
    return fail(PCAST_EINVAL, "order must be 0 (forward) or 1 (reverse)");
  if (Nq <= 0) return fail(PCAST_EINVAL, "Nq must be positive");
  if (Nq > Nk) return fail(PCAST_EINVAL, "Nq = %d exceeds Nk = %d: the rows sit at the last Nq positions", Nq, Nk);
  if (split_keys <= 0 || split_keys % kKvBlock != 0)
    return fail(PCAST_EINVAL, "split_keys must be a positive multiple of %d", kKvBlock);
  int rc = check_shape(B, Hq, Hkv, Nk, d, S, any_nk);
  if (rc != PCAST_OK) return rc;
  if (S == 0.0f) return fail(PCAST_ENOTSUP, "decode needs S > 0 (the FP8 P.V path)");
  if ((int64_t)(Hq / Hkv) * Nq > 32)
    return fail(PCAST_ENOTSUP, "(Hq / Hkv) * Nq = %lld: at most 32 rows per kv head", (long long)(Hq / Hkv) * Nq);
  const DecodeLayout l = decode_layout(B, Hkv, Nk, d, split_keys);
  if ((int64_t)B * Hkv * l.n_split > (int64_t)INT32_MAX) return fail(PCAST_ENOTSUP, "grid too large");
  return check_device();
}

// The decode's two kernels; K as bf16 (K) or as E4M3 codes with block exponents (k8, kexp).
int enqueue_decode(const void* Q, const void* K, const void* vop, const uint8_t* k8, const int* kexp,
                   const float* bias, int B, int Hq, int Hkv, int Nq, int Nk, int d, float S, int order,
                   int split_keys, float* out, unsigned long long* stats, void* workspace, hipStream_t st) {
  const DecodeLayout l = decode_layout(B, Hkv, Nk, d, split_keys);
  Params p{};
  p.q = static_cast<const uint16_t*>(Q);
  p.k = static_cast<const uint16_t*>(K);
  p.k8 = k8;
  p.kexp = kexp;
  p.vop = vop;
  p.bias = bias;
  p.out = out;
  p.stats = stats;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = Nk;
  p.order = order;
  p.logit_scale = (float)(1.4426950408889634 / std::sqrt((double)d));
  p.S = S;
  p.inv_S = 1.0f / S;
  p.p_clamp = 448.0f / S;
  p.Nq = Nq; p.Nk = Nk; p.n_split = l.n_split; p.split_blocks = split_keys / kKvBlock;
  uint8_t* base = static_cast<uint8_t*>(workspace);
  p.part_a = reinterpret_cast<float*>(base + l.a);
  p.part_ml = reinterpret_cast<float*>(base + l.ml);
  p.part_cnt = reinterpret_cast<unsigned int*>(base + l.cnt);
  const int mode = (is_pow2(S) ? kPow2 : kMul) + (S > 448.0f ? 1 : 0);
  const bool qk8 = k8 != nullptr;
  const dim3 grid((unsigned)(B * Hkv * l.n_split)), mgrid((unsigned)(B * Hkv));
#define PCAST_DECODE(DD, MM, Q8)                                                                    \
  do {                                                                                              \
    if (stats) {                                                                                    \
      hipLaunchKernelGGL((pcast_decode_split<DD, MM, true, Q8>), grid, dim3(64), 0, st, p);         \
      hipLaunchKernelGGL((pcast_decode_merge<DD, true>), mgrid, dim3(256), 0, st, p);               \
    } else {                                                                                        \
      hipLaunchKernelGGL((pcast_decode_split<DD, MM, false, Q8>), grid, dim3(64), 0, st, p);        \
      hipLaunchKernelGGL((pcast_decode_merge<DD, false>), mgrid, dim3(256), 0, st, p);              \
    }                                                                                               \
  } while (0)
#define PCAST_DECODE_MODES(DD, Q8)                              \
  switch (mode) {                                               \
    case kPow2: PCAST_DECODE(DD, kPow2, Q8); break;             \
    case kPow2Clamp: PCAST_DECODE(DD, kPow2Clamp, Q8); break;   \
    case kMul: PCAST_DECODE(DD, kMul, Q8); break;               \
    default: PCAST_DECODE(DD, kMulClamp, Q8); break;            \
  }
  if (d == 64) {
    if (qk8) PCAST_DECODE_MODES(64, true) else PCAST_DECODE_MODES(64, false)
  } else {
    if (qk8) PCAST_DECODE_MODES(128, true) else PCAST_DECODE_MODES(128, false)
  }
#undef PCAST_DECODE_MODES
#undef PCAST_DECODE
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PCAST_OK : hip_fail(e, "decode kernel launch");
}

}  // namespace

extern "C" {

int pcast_prepare_v(const void* V, int B, int Hkv, int N, int d, float S, void* workspace,
                    void* stream) {
  g_last_error[0] = '\0';
  if (!V || !workspace) return fail(PCAST_EINVAL, "V and workspace must be non-null");
  if (!aligned(V, 16) || !aligned(workspace, 16))
    return fail(PCAST_EINVAL, "V and workspace must be 16-byte aligned");
  int rc = check_shape(B, Hkv, Hkv, N, d, S, true);
  if (rc != PCAST_OK) return rc;
  if ((rc = check_device()) != PCAST_OK) return rc;
  return enqueue_prep(V, B, Hkv, N, d, S, workspace, static_cast<hipStream_t>(stream));
}

int attn_fwd_pcast_prepared(const void* Q, const void* K, const void* workspace, const float* bias,
                            int B, int Hq, int Hkv, int N, int d, int causal, float S, int order,
                            float* out, unsigned long long* stats, void* stream) {
  g_last_error[0] = '\0';
  if (!workspace) return fail(PCAST_EINVAL, "workspace must be non-null");
  if (!aligned(workspace, 16)) return fail(PCAST_EINVAL, "workspace must be 16-byte aligned");
  int rc = check_attn_args(Q, K, bias, causal, order, out, stats);
  if (rc != PCAST_OK) return rc;
  if ((rc = check_shape(B, Hq, Hkv, N, d, S, true)) != PCAST_OK) return rc;
  if ((rc = check_device()) != PCAST_OK) return rc;
  return enqueue_attn(Q, K, workspace, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats,
                      static_cast<hipStream_t>(stream));
}

int attn_fwd_pcast(const void* Q, const void* K, const void* V, const float* bias, int B, int Hq,
                   int Hkv, int N, int d, int causal, float S, int order, float* out,
                   unsigned long long* stats, void* stream) {
  g_last_error[0] = '\0';
  // ---- argument checks: nothing touches the device before they pass ----
  int rc = check_attn_args(Q, K, bias, causal, order, out, stats);
  if (rc != PCAST_OK) return rc;
  if (!V) return fail(PCAST_EINVAL, "V must be non-null");
  if (!aligned(V, 16)) return fail(PCAST_EINVAL, "V must be 16-byte aligned");
  if ((rc = check_shape(B, Hq, Hkv, N, d, S, true)) != PCAST_OK) return rc;
  if ((rc = check_device()) != PCAST_OK) return rc;

  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, pcast_workspace_bytes(B, Hkv, N, d, S), st);
  if (e != hipSuccess) return hip_fail(e, "hipMallocAsync(workspace)");
  rc = enqueue_prep(V, B, Hkv, N, d, S, ws, st);
  if (rc == PCAST_OK) rc = enqueue_attn(Q, K, ws, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats, st);
  e = hipFreeAsync(ws, st);
  if (rc != PCAST_OK) return rc;
  if (e != hipSuccess) return hip_fail(e, "hipFreeAsync(workspace)");
  return PCAST_OK;
}

int attn_fwd_pcast_noalloc(const void* Q, const void* K, const void* V, const float* bias, int B, int Hq,
                           int Hkv, int N, int d, int causal, float S, int order, float* out,
                           unsigned long long* stats, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_attn_args(Q, K, bias, causal, order, out, stats);
  if (rc != PCAST_OK) return rc;
  if (!V) return fail(PCAST_EINVAL, "V must be non-null");
  if (!aligned(V, 16)) return fail(PCAST_EINVAL, "V must be 16-byte aligned");
  if ((rc = check_shape(B, Hq, Hkv, N, d, S, true)) != PCAST_OK) return rc;
  const size_t need = pcast_workspace_bytes(B, Hkv, N, d, S);
  if (need > (size_t)PCAST_NOALLOC_SCRATCH_BYTES)
    return fail(PCAST_ENOTSUP,
                "the V operand copy needs %zu bytes, above the %zu bytes of scratch of attn_fwd_pcast_noalloc; "
                "use attn_fwd_pcast, or pcast_prepare_v + attn_fwd_pcast_prepared with a caller workspace",
                need, (size_t)PCAST_NOALLOC_SCRATCH_BYTES);
  if ((rc = check_device()) != PCAST_OK) return rc;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws)) != PCAST_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the pre-pass writes every byte of the copy that the attention kernel reads: no clearing
  rc = enqueue_prep(V, B, Hkv, N, d, S, ws, st);
  if (rc == PCAST_OK) rc = enqueue_attn(Q, K, ws, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats, st);
  return rc;
}

int attn_fwd_pcast_multi(const void* Q, const void* K, const void* workspace, int B, int Hq, int Hkv, int N, int d,
                         int causal, int n_cfg, const float* const* bias, const float* S, const int* order,
                         float* const* out, unsigned long long* const* stats, void* stream) {
  g_last_error[0] = '\0';
  if (!Q || !K || !workspace) return fail(PCAST_EINVAL, "Q, K and workspace must be non-null");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(workspace, 16))
    return fail(PCAST_EINVAL, "Q, K and workspace must be 16-byte aligned");
  if (causal != 0 && causal != 1) return fail(PCAST_EINVAL, "causal must be 0 or 1");
  if (n_cfg < 1) return fail(PCAST_EINVAL, "n_cfg = %d: must be positive", n_cfg);
  if (!S || !order || !out) return fail(PCAST_EINVAL, "the S, order and out arrays must be non-null");
  for (int i = 0; i < n_cfg; ++i) {
    if (!out[i] || !aligned(out[i], 16)) return fail(PCAST_EINVAL, "out[%d] must be non-null and 16-byte aligned", i);
    if (bias && bias[i] && !aligned(bias[i], 4)) return fail(PCAST_EINVAL, "bias[%d] must be 4-byte aligned", i);
    if (stats && (!stats[i] || !aligned(stats[i], 8)))
      return fail(PCAST_EINVAL, "stats[%d] must be non-null and 8-byte aligned when stats is given", i);
    if (order[i] != PCAST_ORDER_FORWARD && order[i] != PCAST_ORDER_REVERSE)
      return fail(PCAST_EINVAL, "order[%d] must be 0 (forward) or 1 (reverse)", i);
    if (!std::isfinite(S[i]) || S[i] < 0.0f) return fail(PCAST_EINVAL, "S[%d] must be finite and >= 0", i);
    if (S[i] == 0.0f) return fail(PCAST_ENOTSUP, "S[%d] = 0: the multi-configuration call runs the FP8 P.V path only", i);
  }
  int rc = check_shape(B, Hq, Hkv, N, d, S[0], true);
  if (rc != PCAST_OK) return rc;
  if ((int64_t)B * Hq * ((N + kBlockRows - 1) / kBlockRows) * kMaxCells > (int64_t)INT32_MAX)
    return fail(PCAST_ENOTSUP, "grid too large");
  if ((rc = check_device()) != PCAST_OK) return rc;

  Params p{};
  p.q = static_cast<const uint16_t*>(Q);
  p.k = static_cast<const uint16_t*>(K);
  p.vop = workspace;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N;
  p.logit_scale = (float)(1.4426950408889634 / std::sqrt((double)d));
  hipStream_t st = static_cast<hipStream_t>(stream);
  // one launch per conversion mode and per kMaxCells cells of that mode, the cells of a
  // mode split evenly over its launches (no small last launch draining the chip alone)
  auto mode_of = [&](int i) { return (is_pow2(S[i]) ? kPow2 : kMul) + (S[i] > 448.0f ? 1 : 0); };
  for (int mode = kPow2; mode <= kMulClamp; ++mode) {
    int count = 0;
    for (int i = 0; i < n_cfg; ++i) count += mode_of(i) == mode;
    if (count == 0) continue;
    const int launches = (count + kMaxCells - 1) / kMaxCells;
    const int per_launch = (count + launches - 1) / launches;
    Cells cells{};
    auto flush = [&]() -> int {
      if (cells.n == 0) return PCAST_OK;
      if (d == 64) launch_multi<64>(p, cells, mode, causal, stats != nullptr, st);
      else launch_multi<128>(p, cells, mode, causal, stats != nullptr, st);
      cells.n = 0;
      const hipError_t e = hipGetLastError();
      return e == hipSuccess ? PCAST_OK : hip_fail(e, "multi-configuration attention launch");
    };
    for (int i = 0; i < n_cfg; ++i) {
      if (mode_of(i) != mode) continue;
      const int c = cells.n++;
      cells.bias[c] = bias ? bias[i] : nullptr;
      cells.out[c] = out[i];
      cells.stats[c] = stats ? stats[i] : nullptr;
      cells.S[c] = S[i];
      cells.order[c] = order[i];
      if (cells.n == per_launch && (rc = flush()) != PCAST_OK) return rc;
    }
    if ((rc = flush()) != PCAST_OK) return rc;
  }
  return PCAST_OK;
}

int attn_fwd_pcast_rows(const void* Q, const void* K, const void* workspace, const float* bias, int B,
                        int Hq, int Hkv, int N, int d, int causal, float S, int order, float* out,
                        unsigned long long* stats, float* lse, float* lost, void* stream) {
  g_last_error[0] = '\0';
  if (!workspace) return fail(PCAST_EINVAL, "workspace must be non-null");
  if (!aligned(workspace, 16)) return fail(PCAST_EINVAL, "workspace must be 16-byte aligned");
  int rc = check_attn_args(Q, K, bias, causal, order, out, stats);
  if (rc != PCAST_OK) return rc;
  if ((lse && !aligned(lse, 4)) || (lost && !aligned(lost, 4)))
    return fail(PCAST_EINVAL, "lse and lost must be 4-byte aligned");
  if ((rc = check_shape(B, Hq, Hkv, N, d, S, true)) != PCAST_OK) return rc;
  if (S == 0.0f) return fail(PCAST_ENOTSUP, "row diagnostics need S > 0 (the FP8 P.V path)");
  if ((rc = check_device()) != PCAST_OK) return rc;
  return enqueue_attn(Q, K, workspace, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats,
                      static_cast<hipStream_t>(stream), false, lse, lost);
}

}  // extern "C"

namespace {

// The backward's three launches on N rows (N a multiple of 64 here).
int enqueue_bwd(const void* Q, const void* K, const void* V, const float* O, const void* dO, const float* lse,
                const float* bias, int B, int Hq, int Hkv, int N, int d, int causal, float* dQ, float* dK, float* dV,
                void* workspace, hipStream_t st) {
  const BwdLayout l = bwd_layout(B, Hq, Hkv, N, d);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  const int64_t rows = (int64_t)B * Hq * N;
  const uint16_t* Qb = static_cast<const uint16_t*>(Q);
  const uint16_t* Kb = static_cast<const uint16_t*>(K);
  const uint16_t* dOb = static_cast<const uint16_t*>(dO);
  const float sqrt_d = std::sqrt((float)d);
  float* dvec = reinterpret_cast<float*>(base + l.dvec);
  float* nls = reinterpret_cast<float*>(base + l.nls);
  if (d == 64)
    hipLaunchKernelGGL(pcast_bwd_rowdot<64>, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, st, dOb, O, lse,
                       dvec, nls, sqrt_d, rows);
  else
    hipLaunchKernelGGL(pcast_bwd_rowdot<128>, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, st, dOb, O, lse,
                       dvec, nls, sqrt_d, rows);
  Params p{};
  p.q = Qb;
  p.k = Kb;
  p.v = static_cast<const uint16_t*>(V);
  p.dout = dOb;
  p.lse_in = lse;
  p.dvec = dvec;
  p.nls = nls;
  p.bias = bias;
  p.dq = dQ;
  p.dk = dK;
  p.dv = dV;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N;
  p.logit_scale = (float)(1.4426950408889634 / std::sqrt((double)d));
  const int n_rb = (N + kBlockRows - 1) / kBlockRows, n_qb = (N + kDqRows - 1) / kDqRows;
  const dim3 gq((unsigned)(n_qb * Hq * B)), gk((unsigned)(n_rb * Hkv * B));
  if (d == 64) {
    if (causal) {
      hipLaunchKernelGGL((pcast_attn_bwd_dq<64, true>), gq, dim3(kDqWaves * 64), 0, st, p);
      hipLaunchKernelGGL((pcast_attn_bwd_dkv<64, true>), gk, dim3(kThreads), 0, st, p);
    } else {
      hipLaunchKernelGGL((pcast_attn_bwd_dq<64, false>), gq, dim3(kDqWaves * 64), 0, st, p);
      hipLaunchKernelGGL((pcast_attn_bwd_dkv<64, false>), gk, dim3(kThreads), 0, st, p);
    }
  } else {
    if (causal) {
      hipLaunchKernelGGL((pcast_attn_bwd_dq<128, true>), gq, dim3(kDqWaves * 64), 0, st, p);
      hipLaunchKernelGGL((pcast_attn_bwd_dkv<128, true>), gk, dim3(kThreads), 0, st, p);
    } else {
      hipLaunchKernelGGL((pcast_attn_bwd_dq<128, false>), gq, dim3(kDqWaves * 64), 0, st, p);
      hipLaunchKernelGGL((pcast_attn_bwd_dkv<128, false>), gk, dim3(kThreads), 0, st, p);
    }
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PCAST_OK : hip_fail(e, "backward launch");
}

int fill_u32(void* dst, uint32_t value, int64_t n, hipStream_t st) {
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  if (blocks > 0)
    hipLaunchKernelGGL(pcast_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<uint32_t*>(dst), value, n);
  return hipGetLastError() == hipSuccess ? PCAST_OK : fail(PCAST_EHIP, "fill launch");
}

// rows of `width` bytes from a tensor of `rows` x N rows into one of `rows` x Np rows (and back)
int copy_rows(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t rows, hipStream_t st) {
  const hipError_t e = hipMemcpy2DAsync(dst, dpitch, src, spitch, width, rows, hipMemcpyDeviceToDevice, st);
  return e == hipSuccess ? PCAST_OK : hip_fail(e, "hipMemcpy2DAsync");
}

}  // namespace

extern "C" {

int attn_bwd_pcast(const void* Q, const void* K, const void* V, const float* O, const void* dO,
                   const float* lse, const float* bias, int B, int Hq, int Hkv, int N, int d, int causal,
                   float* dQ, float* dK, float* dV, void* workspace, void* stream) {
  g_last_error[0] = '\0';
  if (!Q || !K || !V || !O || !dO || !lse || !dQ || !dK || !dV || !workspace)
    return fail(PCAST_EINVAL, "Q, K, V, O, dO, lse, dQ, dK, dV and workspace must be non-null");
  const void* a16[] = {Q, K, V, O, dO, dQ, dK, dV, workspace};
  for (const void* ptr : a16)
    if (!aligned(ptr, 16)) return fail(PCAST_EINVAL, "tensors and workspace must be 16-byte aligned");
  if (!aligned(lse, 4) || (bias && !aligned(bias, 4))) return fail(PCAST_EINVAL, "lse and bias must be 4-byte aligned");
  if (causal != 0 && causal != 1) return fail(PCAST_EINVAL, "causal must be 0 or 1");
  int rc = check_shape(B, Hq, Hkv, N, d, 1.0f, true);
  if (rc != PCAST_OK) return rc;
  if ((int64_t)B * Hkv * ((N + kBlockRows - 1) / kBlockRows) > (int64_t)INT32_MAX) return fail(PCAST_ENOTSUP, "grid too large");
  const int Np = (N + kKvBlock - 1) / kKvBlock * kKvBlock;
  if ((int64_t)Np * d * 2 > (int64_t)INT32_MAX)
    return fail(PCAST_ENOTSUP, "N = %d, d = %d: the backward addresses one head's rows with 32-bit byte offsets", N, d);
  if ((rc = check_device()) != PCAST_OK) return rc;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (N % kKvBlock == 0)
    return enqueue_bwd(Q, K, V, O, dO, lse, bias, B, Hq, Hkv, N, d, causal, dQ, dK, dV, workspace, st);
  // a partial last key block: run on whole-block copies (pure data movement around the kernels)
  const BwdPad l = bwd_pad_layout(B, Hq, Hkv, N, d);
  uint8_t* w = static_cast<uint8_t*>(workspace);
  const size_t rq = (size_t)B * Hq, rk = (size_t)B * Hkv;  // heads
  // zeros everywhere (bf16 and fp32 zero are both all-zero bits), then the real rows
  if ((rc = fill_u32(w + l.q, 0u, (int64_t)((l.bias - l.q) / 4), st)) != PCAST_OK) return rc;
  const size_t rowq = (size_t)N * d, padq = (size_t)Np * d;  // elements per head
  if ((rc = copy_rows(w + l.q, padq * 2, Q, rowq * 2, rowq * 2, rq, st)) != PCAST_OK) return rc;
  if ((rc = copy_rows(w + l.k, padq * 2, K, rowq * 2, rowq * 2, rk, st)) != PCAST_OK) return rc;
  if ((rc = copy_rows(w + l.v, padq * 2, V, rowq * 2, rowq * 2, rk, st)) != PCAST_OK) return rc;
  if ((rc = copy_rows(w + l.o, padq * 4, O, rowq * 4, rowq * 4, rq, st)) != PCAST_OK) return rc;
  if ((rc = copy_rows(w + l.dout, padq * 2, dO, rowq * 2, rowq * 2, rq, st)) != PCAST_OK) return rc;
  if ((rc = copy_rows(w + l.lse, (size_t)Np * 4, lse, (size_t)N * 4, (size_t)N * 4, rq, st)) != PCAST_OK) return rc;
  // bias: the caller's (or 0) on the first N keys, -inf on the keys past N
  if ((rc = fill_u32(w + l.bias, 0xFF800000u, Np, st)) != PCAST_OK) return rc;
  if (bias) {
    if ((rc = copy_rows(w + l.bias, (size_t)N * 4, bias, (size_t)N * 4, (size_t)N * 4, 1, st)) != PCAST_OK) return rc;
  } else if ((rc = fill_u32(w + l.bias, 0u, N, st)) != PCAST_OK) {
    return rc;
  }
  rc = enqueue_bwd(w + l.q, w + l.k, w + l.v, reinterpret_cast<const float*>(w + l.o), w + l.dout,
                   reinterpret_cast<const float*>(w + l.lse), reinterpret_cast<const float*>(w + l.bias), B, Hq, Hkv,
                   Np, d, causal, reinterpret_cast<float*>(w + l.dq), reinterpret_cast<float*>(w + l.dk),
                   reinterpret_cast<float*>(w + l.dv), workspace, st);
  if (rc != PCAST_OK) return rc;
  if ((rc = copy_rows(dQ, rowq * 4, w + l.dq, padq * 4, rowq * 4, rq, st)) != PCAST_OK) return rc;
  if ((rc = copy_rows(dK, rowq * 4, w + l.dk, padq * 4, rowq * 4, rk, st)) != PCAST_OK) return rc;
  return copy_rows(dV, rowq * 4, w + l.dv, padq * 4, rowq * 4, rk, st);
}

int attn_decode_pcast(const void* Q, const void* K, const void* vop, const float* bias, int B, int Hq,
                      int Hkv, int Nq, int Nk, int d, float S, int order, int split_keys, float* out,
                      unsigned long long* stats, void* workspace, void* stream) {
  g_last_error[0] = '\0';
  if (!Q || !K || !vop || !out || !workspace)
    return fail(PCAST_EINVAL, "Q, K, vop, out and workspace must be non-null");
  if (!aligned(K, 16) || !aligned(vop, 16))
    return fail(PCAST_EINVAL, "Q, K, vop, out and workspace must be 16-byte aligned");
  const int rc = check_decode(Q, bias, B, Hq, Hkv, Nq, Nk, d, S, order, split_keys, out, stats, workspace, true);
  if (rc != PCAST_OK) return rc;
  return enqueue_decode(Q, K, vop, nullptr, nullptr, bias, B, Hq, Hkv, Nq, Nk, d, S, order, split_keys, out,
                        stats, workspace, static_cast<hipStream_t>(stream));
}

int attn_decode_pcast_qk8(const void* Q, const void* qk8_workspace, const float* bias, int B, int Hq, int Hkv,
                          int Nq, int Nk, int d, float S, int order, int split_keys, float* out,
                          unsigned long long* stats, void* workspace, void* stream) {
  g_last_error[0] = '\0';
  if (!Q || !qk8_workspace || !out || !workspace)
    return fail(PCAST_EINVAL, "Q, qk8_workspace, out and workspace must be non-null");
  if (!aligned(qk8_workspace, 16))
    return fail(PCAST_EINVAL, "Q, qk8_workspace, out and workspace must be 16-byte aligned");
  const int rc = check_decode(Q, bias, B, Hq, Hkv, Nq, Nk, d, S, order, split_keys, out, stats, workspace, true);
  if (rc != PCAST_OK) return rc;
  const Qk8Layout l = qk8_layout(B, Hkv, Nk, d);
  const uint8_t* base = static_cast<const uint8_t*>(qk8_workspace);
  return enqueue_decode(Q, nullptr, qk8_workspace, base + l.k8, reinterpret_cast<const int*>(base + l.kexp), bias,
                        B, Hq, Hkv, Nq, Nk, d, S, order, split_keys, out, stats, workspace,
                        static_cast<hipStream_t>(stream));
}

int pcast_cast_e4m3(const float* P, unsigned char* codes, long long n, float S, void* stream) {
  g_last_error[0] = '\0';
  if (!P || !codes) return fail(PCAST_EINVAL, "P and codes must be non-null");
  if (!aligned(P, 16) || !aligned(codes, 4)) return fail(PCAST_EINVAL, "P must be 16-byte and codes 4-byte aligned");
  if (n < 0 || n % 4 != 0) return fail(PCAST_EINVAL, "n = %lld: must be a non-negative multiple of 4", n);
  if (!std::isfinite(S) || !(S > 0.0f)) return fail(PCAST_EINVAL, "S must be finite and > 0");
  int rc = check_device();
  if (rc != PCAST_OK) return rc;
  if (n == 0) return PCAST_OK;
  Params p{};
  p.S = S;
  p.inv_S = 1.0f / S;
  p.p_clamp = 448.0f / S;
  const int mode = (is_pow2(S) ? kPow2 : kMul) + (S > 448.0f ? 1 : 0);
  const int64_t n4 = n / 4;
  const unsigned blocks = (unsigned)std::min<int64_t>((n4 + 255) / 256, 1 << 16);
  const float4* src = reinterpret_cast<const float4*>(P);
  uint32_t* dst = reinterpret_cast<uint32_t*>(codes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (mode) {
    case kPow2: hipLaunchKernelGGL(pcast_cast_probs<kPow2>, dim3(blocks), dim3(256), 0, st, p, src, dst, n4); break;
    case kPow2Clamp: hipLaunchKernelGGL(pcast_cast_probs<kPow2Clamp>, dim3(blocks), dim3(256), 0, st, p, src, dst, n4); break;
    case kMul: hipLaunchKernelGGL(pcast_cast_probs<kMul>, dim3(blocks), dim3(256), 0, st, p, src, dst, n4); break;
    default: hipLaunchKernelGGL(pcast_cast_probs<kMulClamp>, dim3(blocks), dim3(256), 0, st, p, src, dst, n4); break;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PCAST_OK : hip_fail(e, "cast kernel launch");
}

int pcast_prepare_qk8_rot(const void* Q, const void* K, const void* V, const signed char* signs, int B, int Hq,
                          int Hkv, int N, int d, void* workspace, void* stream) {
  g_last_error[0] = '\0';
  if (!Q || !K || !V || !signs || !workspace) return fail(PCAST_EINVAL, "Q, K, V, signs and workspace must be non-null");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(signs, 16) || !aligned(workspace, 16))
    return fail(PCAST_EINVAL, "Q, K, V, signs and workspace must be 16-byte aligned");
  int rc = check_shape(B, Hq, Hkv, N, d, 1.0f, true);
  if (rc != PCAST_OK) return rc;
  if ((rc = check_device()) != PCAST_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Qk8Layout l = qk8_layout(B, Hkv, N, d, Hq);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  const uint16_t* Qb = static_cast<const uint16_t*>(Q);
  const uint16_t* Kb = static_cast<const uint16_t*>(K);
  const int n_tiles = (N + kKvBlock - 1) / kKvBlock;
  const int64_t qblk = (int64_t)B * Hq * n_tiles, kblk = (int64_t)B * Hkv * n_tiles;
  if ((rc = enqueue_prep(V, B, Hkv, N, d, 1.0f, workspace, st)) != PCAST_OK) return rc;
  int* kexp = reinterpret_cast<int*>(base + l.kexp);
  int* qexp = reinterpret_cast<int*>(base + l.qexp);
  if (d == 64) {
    hipLaunchKernelGGL((pcast_prep_rot8<64, false>), dim3((unsigned)kblk), dim3(256), 0, st, Kb, signs, base + l.k8, kexp,
                       N, n_tiles);
    hipLaunchKernelGGL((pcast_prep_rot8<64, true>), dim3((unsigned)qblk), dim3(256), 0, st, Qb, signs, base + l.q8, qexp,
                       N, n_tiles);
  } else {
    hipLaunchKernelGGL((pcast_prep_rot8<128, false>), dim3((unsigned)kblk), dim3(256), 0, st, Kb, signs, base + l.k8, kexp,
                       N, n_tiles);
    hipLaunchKernelGGL((pcast_prep_rot8<128, true>), dim3((unsigned)qblk), dim3(256), 0, st, Qb, signs, base + l.q8, qexp,
                       N, n_tiles);
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PCAST_OK : hip_fail(e, "rotation pre-pass launch");
}

int attn_fwd_pcast_qk8_rot_prepared(const void* workspace, const float* bias, int B, int Hq, int Hkv, int N, int d,
                                    int causal, float S, int order, float* out, unsigned long long* stats,
                                    void* stream) {
  g_last_error[0] = '\0';
  if (!workspace) return fail(PCAST_EINVAL, "workspace must be non-null");
  if (!aligned(workspace, 16)) return fail(PCAST_EINVAL, "workspace must be 16-byte aligned");
  int rc = check_attn_args(workspace, workspace, bias, causal, order, out, stats);
  if (rc != PCAST_OK) return rc;
  if ((rc = check_shape(B, Hq, Hkv, N, d, S, true)) != PCAST_OK) return rc;
  if ((rc = check_qk8(S)) != PCAST_OK) return rc;
  if ((rc = check_device()) != PCAST_OK) return rc;
  return enqueue_attn(nullptr, nullptr, workspace, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats,
                      static_cast<hipStream_t>(stream), true, nullptr, nullptr, true);
}

int pcast_prepare_qk8(const void* K, const void* V, int B, int Hkv, int N, int d, void* workspace,
                      void* stream) {
  g_last_error[0] = '\0';
  if (!K || !V || !workspace) return fail(PCAST_EINVAL, "K, V and workspace must be non-null");
  if (!aligned(K, 16) || !aligned(V, 16) || !aligned(workspace, 16))
    return fail(PCAST_EINVAL, "K, V and workspace must be 16-byte aligned");
  int rc = check_shape(B, Hkv, Hkv, N, d, 1.0f, true);
  if (rc != PCAST_OK) return rc;
  if ((rc = check_device()) != PCAST_OK) return rc;
  return enqueue_prep_qk8(K, V, B, Hkv, N, d, workspace, static_cast<hipStream_t>(stream));
}

int attn_fwd_pcast_qk8_prepared(const void* Q, const void* workspace, const float* bias, int B, int Hq,
                                int Hkv, int N, int d, int causal, float S, int order, float* out,
                                unsigned long long* stats, void* stream) {
  g_last_error[0] = '\0';
  if (!workspace) return fail(PCAST_EINVAL, "workspace must be non-null");
  if (!aligned(workspace, 16)) return fail(PCAST_EINVAL, "workspace must be 16-byte aligned");
  int rc = check_attn_args(Q, workspace, bias, causal, order, out, stats);
  if (rc != PCAST_OK) return rc;
  if ((rc = check_shape(B, Hq, Hkv, N, d, S, true)) != PCAST_OK) return rc;
  if ((rc = check_qk8(S)) != PCAST_OK) return rc;
  if ((rc = check_device()) != PCAST_OK) return rc;
  return enqueue_attn(Q, nullptr, workspace, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats,
                      static_cast<hipStream_t>(stream), true);
}

int attn_fwd_pcast_qk8(const void* Q, const void* K, const void* V, const float* bias, int B, int Hq,
                       int Hkv, int N, int d, int causal, float S, int order, float* out,
                       unsigned long long* stats, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_attn_args(Q, K, bias, causal, order, out, stats);
  if (rc != PCAST_OK) return rc;
  if (!V) return fail(PCAST_EINVAL, "V must be non-null");
  if (!aligned(V, 16)) return fail(PCAST_EINVAL, "V must be 16-byte aligned");
  if ((rc = check_shape(B, Hq, Hkv, N, d, S, true)) != PCAST_OK) return rc;
  if ((rc = check_qk8(S)) != PCAST_OK) return rc;
  if ((rc = check_device()) != PCAST_OK) return rc;

  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, pcast_workspace_bytes_qk8(B, Hkv, N, d), st);
  if (e != hipSuccess) return hip_fail(e, "hipMallocAsync(workspace)");
  rc = enqueue_prep_qk8(K, V, B, Hkv, N, d, ws, st);
  if (rc == PCAST_OK)
    rc = enqueue_attn(Q, nullptr, ws, bias, B, Hq, Hkv, N, d, causal, S, order, out, stats, st, true);
  e = hipFreeAsync(ws, st);
  if (rc != PCAST_OK) return rc;
  if (e != hipSuccess) return hip_fail(e, "hipFreeAsync(workspace)");
  return PCAST_OK;
}

}  // extern "C"
