// FP8 "P-cast" attention forward for MI355X (gfx950 / CDNA4).
//
// What is computed (FlashAttention blog, "L'algoritmo Flash Attention" and
// "La ricorrenza softmax online"; P-cast summaries, sections 1-2): for every
// query row, key blocks of 64 are visited forward or in reverse; the running
// max m' includes the current block; P = exp(s - m') is summed un-cast into l;
// P*S is rounded to E4M3 and multiplied with E4M3(V) on the FP8 matrix cores;
// the accumulator is rescaled by exp(m - m') when the max grows and divided by
// S*l at the end.  S = 0 runs the same pipeline with P and V in bf16.
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
// * K and V tiles are staged through LDS, double-buffered: the global loads
//   of block j+1 are in flight while block j is computed.
// * Exactness of the scale: for S = 2^k the product P*S is formed inside the
//   conversion (v_cvt_scalef32_pk_fp8_f32 with scale 2^-k), which is exact;
//   1/(S*l) is exact up to the final reciprocal.  Other S use an fp32 multiply
//   (not exact, as the P-cast summary notes for 448), and S > 448 clamps first
//   because the conversion does not saturate by itself.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "pcast_attn.h"

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

// Key (within a 64-key block) held by lane group g (= lane / 32) in operand
// slot b (0..31).  It is the order of the S^T accumulator: register r of
// accumulator kb holds key kb*32 + (r/4)*8 + g*4 + r%4, and slot b = kb*16 + r.
__host__ __device__ constexpr int slot_key(int g, int b) {
  return (b >> 4) * 32 + ((b & 15) >> 2) * 8 + g * 4 + (b & 3);
}

template <int D>
struct Geometry {
  static constexpr int kKStride = D * 2 + 16;  // bytes per K row in LDS (padded)
  static constexpr int kQSteps = D / 16;       // bf16 MFMA k-steps over d
  static constexpr int kDTiles = D / 32;       // 32-column output tiles
};

// ---------------------------------------------------------------------------
// Pre-pass: V (bf16, [B][Hkv][N][D]) -> operand copy [B][Hkv][N/64][D][64]
// in slot order, E4M3 (RNE, saturating) or bf16.
// ---------------------------------------------------------------------------
template <int D, bool kFp8>
__global__ __launch_bounds__(256) void pcast_prep_v(const uint16_t* __restrict__ V,
                                                     void* __restrict__ vop) {
  __shared__ uint16_t tile[kKvBlock][D + 2];
  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;  // flat (b, hkv, key block)
  const uint16_t* src = V + blk * kKvBlock * D;
  for (int c = tid; c < kKvBlock * D / 8; c += 256) {
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    const i32x4_t v = *reinterpret_cast<const i32x4_t*>(src + row * D + col);
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

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const void* vop;
  const float* bias;
  float* out;
  unsigned long long* stats;
  int B, Hq, Hkv, N;
  int causal, order;
  float logit_scale;  // log2(e) / sqrt(d)
  float S;            // P-cast scale (1 in the bf16 path)
  float inv_S;        // 1/S, the conversion scale when S is a power of two
  float p_clamp;      // largest P kept before conversion (448/S when S > 448)
  int scale_mode;     // 0: S = 2^k <= 448, 1: S = 2^k > 448, 2: other S <= 448, 3: other S > 448
};

__device__ inline uint32_t zero_bytes(uint32_t w) {
  const uint32_t t = (w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;
  return __builtin_popcount(~(t | w | 0x7F7F7F7Fu));
}

__device__ inline uint32_t zero_halves(uint32_t w) {
  return ((w & 0xFFFFu) == 0) + ((w >> 16) == 0);
}

// Convert 4 probabilities to 4 E4M3 codes in one word.
__device__ inline uint32_t cast4_fp8(const Params& p, float a, float b, float c, float d) {
  if (p.scale_mode & 1) {  // S > 448: keep S*P <= 448
    const float lim = p.p_clamp;
    a = fminf(a, lim); b = fminf(b, lim); c = fminf(c, lim); d = fminf(d, lim);
  }
  if (p.scale_mode < 2) {  // power of two: exact scaling inside the conversion
    s16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2_t{0, 0}, a, b, p.inv_S, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c, d, p.inv_S, true);
    return __builtin_bit_cast(uint32_t, r);
  }
  const float S = p.S;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a * S, b * S, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c * S, d * S, w, true);
  return (uint32_t)w;
}

__device__ inline uint32_t cast2_bf16(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

template <int D, bool kFp8, bool kStats>
__global__ __launch_bounds__(kThreads, 2) void pcast_attn_fwd(const Params p) {
  using G = Geometry<D>;
  constexpr int kEsize = kFp8 ? 1 : 2;                      // bytes per V operand element
  constexpr int kVStride = kKvBlock * kEsize + 16;          // bytes per V^T row in LDS (padded)
  constexpr int kKBytes = kKvBlock * G::kKStride;
  constexpr int kVBytes = D * kVStride;
  constexpr int kKChunks = kKvBlock * D * 2 / 16;           // 16-byte chunks per K block
  constexpr int kVChunks = D * kKvBlock * kEsize / 16;      // 16-byte chunks per V block
  constexpr int kKPer = kKChunks / kThreads;
  constexpr int kVPer = kVChunks / kThreads;
  static_assert(kKChunks % kThreads == 0 && kVChunks % kThreads == 0, "staging split");

  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][kKBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[2][kVBytes];
  __shared__ float lds_bias[2][kKvBlock];  // bias * log2(e) of the staged key block
  __shared__ int lds_bflag[2];              // any non-zero bias in the staged block
  __shared__ unsigned int lds_cnt[2][2];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int g = lane / 32, li = lane % 32;
  const int n_rb = (p.N + kBlockRows - 1) / kBlockRows;
  // causal: heaviest row blocks first
  const int rb = p.causal ? (n_rb - 1 - (int)blockIdx.x) : (int)blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (p.Hq / p.Hkv);
  const int n_tiles = p.N / kKvBlock;
  const int row0 = rb * kBlockRows;
  const int wrow0 = row0 + wave * kRowsPerWave;  // first row of this wave
  const int myrow = wrow0 + li;
  const bool wave_active = wrow0 < p.N;
  const int t_last = p.causal ? min((row0 + kBlockRows - 1) / kKvBlock, n_tiles - 1) : n_tiles - 1;
  const int n_it = t_last + 1;

  if (kStats && tid < 4) lds_cnt[tid / 2][tid % 2] = 0;

  // Q operand (B of S^T = K Q^T): lane holds Q[myrow][s*16 + g*8 .. +8) for each step s.
  bf16x8_t qf[G::kQSteps];
  if (wave_active) {
    const uint16_t* qrow = p.q + (((int64_t)b * p.Hq + h) * p.N + myrow) * D + g * 8;
#pragma unroll
    for (int s = 0; s < G::kQSteps; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + s * 16);
  }

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k + ((int64_t)b * p.Hkv + hk) * p.N * D);
  const uint8_t* vbase = static_cast<const uint8_t*>(p.vop) +
                         ((int64_t)b * p.Hkv + hk) * (int64_t)n_tiles * kKvBlock * D * kEsize;

  i32x4_t kreg[kKPer], vreg[kVPer];
  float breg = 0.0f;
  const bool with_bias = p.bias != nullptr;
  auto tile_of = [&](int it) { return p.order ? (t_last - it) : it; };
  auto load_regs = [&](int t) {
    const uint8_t* ks = kbase + (int64_t)t * kKvBlock * D * 2;
    const uint8_t* vs = vbase + (int64_t)t * kKvBlock * D * kEsize;
#pragma unroll
    for (int i = 0; i < kKPer; ++i) kreg[i] = *reinterpret_cast<const i32x4_t*>(ks + (int64_t)(i * kThreads + tid) * 16);
#pragma unroll
    for (int i = 0; i < kVPer; ++i) vreg[i] = *reinterpret_cast<const i32x4_t*>(vs + (int64_t)(i * kThreads + tid) * 16);
    if (with_bias && wave == 0) breg = p.bias[t * kKvBlock + lane];
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kKPer; ++i) {
      const int c = i * kThreads + tid;
      const int row = c / (D * 2 / 16), part = c % (D * 2 / 16);
      *reinterpret_cast<i32x4_t*>(&lds_k[buf][row * G::kKStride + part * 16]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
      const int c = i * kThreads + tid;
      const int row = c / (kKvBlock * kEsize / 16), part = c % (kKvBlock * kEsize / 16);
      *reinterpret_cast<i32x4_t*>(&lds_v[buf][row * kVStride + part * 16]) = vreg[i];
    }
    if (with_bias && wave == 0) {
      lds_bias[buf][lane] = breg * kLog2e;
      const bool any = __ballot(breg != 0.0f) != 0;
      if (lane == 0) lds_bflag[buf] = any ? 1 : 0;
    }
  };

  f32x16_t oacc[G::kDTiles];
#pragma unroll
  for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  unsigned int cnt_tot = 0, cnt_zero = 0;

  load_regs(tile_of(0));
  store_lds(0);
  __syncthreads();

  for (int it = 0; it < n_it; ++it) {
    const int t = tile_of(it);
    const int cur = it & 1;
    if (it + 1 < n_it) load_regs(tile_of(it + 1));

    const int key0 = t * kKvBlock;
    const bool visible = wave_active && (!p.causal || key0 <= wrow0 + kRowsPerWave - 1);
    if (visible) {
      const bool diag = p.causal && (key0 + kKvBlock - 1 > wrow0);
      const bool has_bias = with_bias && lds_bflag[cur] != 0;
      const float* bl = lds_bias[cur];

      // ---- S^T = K Q^T (two 32-key halves) ----
      f32x16_t sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
      const uint8_t* kl = lds_k[cur];
#pragma unroll
      for (int s = 0; s < G::kQSteps; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kl + (kb * 32 + li) * G::kKStride + (s * 16 + g * 8) * 2);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
        }
      }

      // ---- logits in log2 units, bias, causal mask ----
      float x[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[kb * 16 + r] = sacc[kb][r] * p.logit_scale;
      if (has_bias) {
#pragma unroll
        for (int j = 0; j < 32; ++j) x[j] += bl[slot_key(g, j)];
      }
      if (diag) {
#pragma unroll
        for (int j = 0; j < 32; ++j)
          if (key0 + slot_key(g, j) > myrow) x[j] = -INFINITY;
      }

      // ---- running max (this block included) ----
      float mu = x[0];
#pragma unroll
      for (int j = 1; j < 32; ++j) mu = fmaxf(mu, x[j]);
      mu = fmaxf(mu, __shfl_xor(mu, 32));
      const float m_new = fmaxf(m_run, mu);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);

      // ---- P = exp2(x - m'), row sum from the un-cast P ----
      float psum = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        x[j] = __builtin_amdgcn_exp2f(x[j] - m_use);
        psum += x[j];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;

      // ---- rescale O when any row's max grew (alpha == 1 is an exact no-op) ----
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      }

      if constexpr (kFp8) {
        // ---- P-cast: 32 codes = 8 words, slot order ----
        uint32_t pw[8];
#pragma unroll
        for (int w = 0; w < 8; ++w)
          pw[w] = cast4_fp8(p, x[4 * w], x[4 * w + 1], x[4 * w + 2], x[4 * w + 3]);
        if constexpr (kStats) {
          if (!has_bias && !diag) {
            cnt_tot += 32;
#pragma unroll
            for (int w = 0; w < 8; ++w) cnt_zero += zero_bytes(pw[w]);
          } else {
#pragma unroll
            for (int j = 0; j < 32; ++j) {
              const int key = key0 + slot_key(g, j);
              const bool vis = !p.causal || key <= myrow;
              const bool nonsink = !has_bias || bl[key - key0] == 0.0f;
              const bool z = ((pw[j / 4] >> (8 * (j % 4))) & 0xFFu) == 0;
              cnt_tot += (vis && nonsink);
              cnt_zero += (vis && nonsink && z);
            }
          }
        }
        i32x8_t pb;
#pragma unroll
        for (int w = 0; w < 8; ++w) pb[w] = (int)pw[w];
        // ---- O^T += V8^T P8^T ----
        const uint8_t* vl = lds_v[cur];
#pragma unroll
        for (int dt = 0; dt < G::kDTiles; ++dt) {
          const uint8_t* src = vl + (dt * 32 + li) * kVStride + g * 32;
          const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(src);
          const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(src + 16);
          const i32x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, oacc[dt], 0, 0, 0, 0, 0, 0);
        }
      } else {
        // ---- bf16 path: P in bf16, 4 k-steps of 16 slots ----
        uint32_t pw[16];
#pragma unroll
        for (int w = 0; w < 16; ++w) pw[w] = cast2_bf16(x[2 * w], x[2 * w + 1]);
        if constexpr (kStats) {
#pragma unroll
          for (int j = 0; j < 32; ++j) {
            const int key = key0 + slot_key(g, j);
            const bool vis = !p.causal || key <= myrow;
            const bool nonsink = !has_bias || bl[key - key0] == 0.0f;
            const bool z = ((pw[j / 2] >> (16 * (j % 2))) & 0xFFFFu) == 0;
            cnt_tot += (vis && nonsink);
            cnt_zero += (vis && nonsink && z);
          }
        }
        const uint8_t* vl = lds_v[cur];
#pragma unroll
        for (int dt = 0; dt < G::kDTiles; ++dt) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vl + (dt * 32 + li) * kVStride + (g * 32 + s * 8) * 2);
            i32x4_t bw = {(int)pw[4 * s], (int)pw[4 * s + 1], (int)pw[4 * s + 2], (int)pw[4 * s + 3]};
            const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, bw);
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, oacc[dt], 0, 0, 0);
          }
        }
      }
    }

    if (it + 1 < n_it) store_lds(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = A / (S l) ----
  if (wave_active) {
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / (p.S * l_tot);
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
    unsigned int a = cnt_tot, z = cnt_zero;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      a += __shfl_xor(a, off);
      z += __shfl_xor(z, off);
    }
    if (lane == 0 && wave_active) {
      atomicAdd(&lds_cnt[wave / 2][0], a);
      atomicAdd(&lds_cnt[wave / 2][1], z);
    }
    __syncthreads();
    if (tid < 2) {
      const int r64 = row0 / kKvBlock + tid;  // 64-row block index
      if (r64 * kKvBlock < p.N) {
        unsigned long long* st = p.stats + 2 * (((int64_t)b * p.Hq + h) * (p.N / kKvBlock) + r64);
        st[0] = lds_cnt[tid][0];
        st[1] = lds_cnt[tid][1];
      }
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

bool is_pow2(float S) {
  int e;
  return std::frexp(S, &e) == 0.5f;
}

template <int D, bool kFp8>
void launch_prep(const uint16_t* V, void* ws, int64_t n_blocks, hipStream_t stream) {
  hipLaunchKernelGGL((pcast_prep_v<D, kFp8>), dim3((unsigned)n_blocks), dim3(256), 0, stream, V, ws);
}

template <int D, bool kFp8>
void launch_attn(const Params& p, hipStream_t stream) {
  const dim3 grid((p.N + kBlockRows - 1) / kBlockRows, p.Hq, p.B);
  if (p.stats)
    hipLaunchKernelGGL((pcast_attn_fwd<D, kFp8, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((pcast_attn_fwd<D, kFp8, false>), grid, dim3(kThreads), 0, stream, p);
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

}  // namespace

extern "C" {

size_t pcast_stats_words(int B, int Hq, int N) {
  if (B <= 0 || Hq <= 0 || N <= 0) return 0;
  return (size_t)B * Hq * ((N + kKvBlock - 1) / kKvBlock) * 2;
}

size_t pcast_workspace_bytes(int B, int Hkv, int N, int d, float S) {
  if (B <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return 0;
  return (size_t)B * Hkv * N * d * ((S == 0.0f) ? 2 : 1);
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
int check_shape(int B, int Hq, int Hkv, int N, int d, float S) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0)
    return fail(PCAST_EINVAL, "B, Hq, Hkv, N, d must be positive");
  if (Hq % Hkv != 0) return fail(PCAST_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (!std::isfinite(S) || S < 0.0f) return fail(PCAST_EINVAL, "S must be finite and >= 0");
  if (d != 64 && d != 128) return fail(PCAST_ENOTSUP, "d = %d: supported head sizes are 64 and 128", d);
  if (N % kKvBlock != 0) return fail(PCAST_ENOTSUP, "N = %d: must be a multiple of %d", N, kKvBlock);
  if ((int64_t)B * Hkv * (N / kKvBlock) > (int64_t)INT32_MAX || Hq > 65535 || B > 65535)
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
  const int64_t n_blocks = (int64_t)B * Hkv * (N / kKvBlock);
  const uint16_t* Vb = static_cast<const uint16_t*>(V);
  if (d == 64) {
    if (fp8) launch_prep<64, true>(Vb, ws, n_blocks, st); else launch_prep<64, false>(Vb, ws, n_blocks, st);
  } else {
    if (fp8) launch_prep<128, true>(Vb, ws, n_blocks, st); else launch_prep<128, false>(Vb, ws, n_blocks, st);
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PCAST_OK : hip_fail(e, "V pre-pass launch");
}

int enqueue_attn(const void* Q, const void* K, const void* ws, const float* bias, int B, int Hq,
                 int Hkv, int N, int d, int causal, float S, int order, float* out,
                 unsigned long long* stats, hipStream_t st) {
  const bool fp8 = S != 0.0f;
  Params p{};
  p.q = static_cast<const uint16_t*>(Q);
  p.k = static_cast<const uint16_t*>(K);
  p.vop = ws;
  p.bias = bias;
  p.out = out;
  p.stats = stats;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N;
  p.causal = causal; p.order = order;
  p.logit_scale = (float)(1.4426950408889634 / std::sqrt((double)d));
  p.S = fp8 ? S : 1.0f;
  p.inv_S = fp8 ? 1.0f / S : 1.0f;
  // S > 448: P is clamped to 448/S so that S*P stays at or below 448 (exact for S = 2^k;
  // otherwise S*fl(448/S) may exceed 448 by an ulp, which still rounds to 448).
  p.p_clamp = fp8 ? 448.0f / S : 1.0f;
  p.scale_mode = fp8 ? ((is_pow2(S) ? 0 : 2) | (S > 448.0f ? 1 : 0)) : 0;
  if (d == 64) {
    if (fp8) launch_attn<64, true>(p, st); else launch_attn<64, false>(p, st);
  } else {
    if (fp8) launch_attn<128, true>(p, st); else launch_attn<128, false>(p, st);
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PCAST_OK : hip_fail(e, "attention kernel launch");
}

}  // namespace

extern "C" {

int pcast_prepare_v(const void* V, int B, int Hkv, int N, int d, float S, void* workspace,
                    void* stream) {
  g_last_error[0] = '\0';
  if (!V || !workspace) return fail(PCAST_EINVAL, "V and workspace must be non-null");
  if (!aligned(V, 16) || !aligned(workspace, 16))
    return fail(PCAST_EINVAL, "V and workspace must be 16-byte aligned");
  int rc = check_shape(B, Hkv, Hkv, N, d, S);
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
  if ((rc = check_shape(B, Hq, Hkv, N, d, S)) != PCAST_OK) return rc;
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
  if ((rc = check_shape(B, Hq, Hkv, N, d, S)) != PCAST_OK) return rc;
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

}  // extern "C"
