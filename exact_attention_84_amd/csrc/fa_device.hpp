// Device building blocks of the fused attention forward on gfx950 (CDNA4).
//
// One wavefront owns NT groups of 32 query rows.  Scores are computed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16
// head-dim values read from LDS, B = Q^T held in registers for the whole key
// loop).  In the 32x32 accumulator layout lane l holds query column l % 32
// and 16 key rows {(v & 3) + 8 (v >> 2) + 4 (l >> 5)}, so every lane owns one
// query: the row max and row sum are in-lane, plus one exchange between the
// two half-waves.  The probabilities P^T then already sit in the B-operand
// layout of the second product O^T = V^T P^T, up to a fixed permutation of
// the keys inside each group of 16, which the V^T tile in LDS is stored with.
// So P goes from the exp unit to the matrix core without touching LDS.
//
// Online softmax ("推理优化 | FlashAttention 1-4 详解", section Online Softmax
// 数学推导, update equations): m_new = max(m, rowmax S); P = exp(S - m_new);
// l = exp(m - m_new) l + rowsum P; O = exp(m - m_new) O + P V; O / l at the
// end (deferred normalisation, same page, section 减少非矩阵乘运算占比).  All of
// it runs in base 2 with log2(e) folded into the score scale, so each
// probability costs one FMA and one v_exp_f32 ("FlashAttention — IO 感知的精确
// 注意力 kernel", section 4, the exp2 trick).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round two fp32 values to bf16 (nearest-even) and pack them (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  u32x4 u = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
             pack_bf16x2(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, u);
}

// Max / sum of a value across the two half-waves (lanes l and l ^ 32).
__device__ __forceinline__ float halfwave_max(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float halfwave_sum(float x) { return x + __shfl_xor(x, 32); }

// Key index (within a 32-key sub-tile) of accumulator element v of a lane in
// half-wave hh, for the 32x32 MFMA output layout.
__device__ __forceinline__ int acc_row(int v, int hh) { return (v & 3) + 8 * (v >> 2) + 4 * hh; }

// Position of key k inside its group of 16 in the V^T tile: bits 2 and 3
// swapped.  With it, the eight keys a lane contributes to one 16-key step of
// the P V product are contiguous in LDS.
__device__ __forceinline__ int swap_bits23(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// XOR swizzle of the 16-byte chunks of V^T row d.  Eight consecutive rows
// (one MFMA operand read) and sixteen rows eight apart (one transposing
// store) both fall on distinct bank groups.
__device__ __forceinline__ int vt_swizzle(int d) { return (d & 7) ^ ((d >> 3) & 7); }

// Workgroup id -> work-item id so that consecutive work items run on the same
// XCD (MI355X hands workgroups to its 8 XCDs round-robin).  Consecutive items
// share K/V, which then stays in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = w & 7, slot = w >> 3;
  const int base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return base + slot;
}

// ---------------------------------------------------------------------------
// Cooperative K / V tile staging: global -> registers -> LDS.
//
// K tile: [BC][D + 8] bf16, row-major, 16 bytes of padding per row so that
//         the 32 rows of one MFMA operand read fall on distinct banks.
// V tile: stored transposed, V^T [D][BC], with the key permutation above and
//         the XOR chunk swizzle, so that an A operand of O^T = V^T P^T is one
//         16-byte LDS read per lane.
// Each thread moves whole 16-byte chunks; for V it takes two adjacent keys of
// the same chunk and interleaves them into 32-bit (key, key+1) pairs.
// ---------------------------------------------------------------------------
template <int D, int BC, int T>
struct TileLoader {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int KSTR = D + 8;                // K row stride, elements
  static constexpr int NK = (BC * CPR + T - 1) / T;  // K chunks per thread
  static constexpr int NV = ((BC / 2) * CPR + T - 1) / T;  // V chunk pairs per thread
  static constexpr int K_ELEMS = BC * KSTR;
  static constexpr int VT_ELEMS = D * BC;
  static_assert(BC % 32 == 0 && BC >= 64, "V^T swizzle needs >= 8 chunks per row");

  u32x4 kr[NK];
  u32x4 vr[NV][2];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ kbase,
                                       const uint16_t* __restrict__ vbase, size_t row_stride,
                                       int k0, int kend, int tid) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int c = tid + i * T;
      const int row = c / CPR, col = c % CPR;
      const int key = k0 + row;
      kr[i] = (c < BC * CPR && key < kend)
                  ? *reinterpret_cast<const u32x4*>(kbase + (size_t)key * row_stride + col * 8)
                  : zero;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int pc = tid + i * T;
      const int j = pc / CPR, col = pc % CPR;
      const int key = k0 + swap_bits23(2 * j);
      const bool in = pc < (BC / 2) * CPR;
      vr[i][0] = (in && key < kend)
                     ? *reinterpret_cast<const u32x4*>(vbase + (size_t)key * row_stride + col * 8)
                     : zero;
      vr[i][1] = (in && key + 1 < kend)
                     ? *reinterpret_cast<const u32x4*>(vbase + (size_t)(key + 1) * row_stride +
                                                       col * 8)
                     : zero;
    }
  }

  __device__ __forceinline__ void store(uint16_t* __restrict__ k_lds, uint16_t* __restrict__ vt_lds,
                                        int tid) const {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int c = tid + i * T;
      if (c < BC * CPR) {
        const int row = c / CPR, col = c % CPR;
        *reinterpret_cast<u32x4*>(k_lds + row * KSTR + col * 8) = kr[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int pc = tid + i * T;
      if (pc < (BC / 2) * CPR) {
        const int j = pc / CPR, col = pc % CPR;
        uint32_t* vt32 = reinterpret_cast<uint32_t*>(vt_lds);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t a = vr[i][0][e >> 1], b = vr[i][1][e >> 1];
          const uint32_t pair = (e & 1) ? ((a >> 16) | (b & 0xFFFF0000u))
                                        : ((a & 0xFFFFu) | (b << 16));
          const int d = col * 8 + e;
          const int chunk = (j >> 2) ^ vt_swizzle(d);
          vt32[d * (BC / 2) + chunk * 4 + (j & 3)] = pair;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Per-wave attention state and the three steps of one key tile.
// ---------------------------------------------------------------------------
template <int D, int NT>
struct WaveState {
  bf16x8 qf[NT][D / 16];    // Q^T, B operand of S^T = K Q^T
  f32x16 o[NT][D / 32];     // O^T accumulator (unnormalised)
  float mc[NT];             // running max of the scores, times c = scale*log2(e)
  float l[NT];              // running sum of exp2 over this half-wave's keys

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      mc[t] = -INFINITY;
      l[t] = 0.f;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[t][dt][v] = 0.f;
    }
  }
};

// S^T sub-tile: keys kt*32..kt*32+31 of the LDS K tile against the wave's
// NT query groups.
template <int D, int NT, int KSTR>
__device__ __forceinline__ void scores_subtile(f32x16 (&s)[NT], const uint16_t* __restrict__ k_lds,
                                               int kt, const bf16x8 (&qf)[NT][D / 16], int m32,
                                               int hh) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) s[t][v] = 0.f;
  const uint16_t* krow = k_lds + (kt * 32 + m32) * KSTR + 8 * hh;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * st);
#pragma unroll
    for (int t = 0; t < NT; ++t) s[t] = mfma_32x32x16(a, qf[t][st], s[t]);
  }
}

// Online-softmax update for NKT score sub-tiles: new running max, rescale
// factor, probabilities (fp32 for the row sum, bf16 for the P V product).
template <int D, int NT, int NKT>
__device__ __forceinline__ void softmax_update(WaveState<D, NT>& st, f32x16 (&s)[NKT][NT],
                                               bf16x8 (&pb)[NKT][NT][2], float c) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kt][t][v]);
    mx = halfwave_max(mx);
    const float mnew = fmaxf(st.mc[t], mx * c);
    // A row that has seen only masked keys keeps m = -inf; subtract 0 then so
    // that exp2(-inf - 0) = 0 instead of NaN.
    const float msub = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = fast_exp2(st.mc[t] - msub);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(s[kt][t][8 * u + e], c, -msub));
          rs += p[e];
        }
        pb[kt][t][u] = pack_bf16x8(p);
      }
    st.l[t] = alpha * st.l[t] + rs;
    st.mc[t] = mnew;
    // Rescale the accumulator only when some row's max moved (alpha != 1);
    // skipping alpha == 1 is exact.
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) st.o[t][dt][v] *= alpha;
    }
  }
}

// O^T += V^T P^T for keys kt*32..kt*32+31 of the LDS V^T tile (row stride BC).
template <int D, int NT, int BC>
__device__ __forceinline__ void pv_subtile(WaveState<D, NT>& st, const uint16_t* __restrict__ vt_lds,
                                           int kt, const bf16x8 (&pb)[NT][2], int m32, int hh) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int d = dt * 32 + m32;
    const int sw = vt_swizzle(d);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int chunk = (kt * 4 + 2 * u + hh) ^ sw;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt_lds + d * BC + chunk * 8);
#pragma unroll
      for (int t = 0; t < NT; ++t) st.o[t][dt] = mfma_32x32x16(a, pb[t][u], st.o[t][dt]);
    }
  }
}

}  // namespace fa
