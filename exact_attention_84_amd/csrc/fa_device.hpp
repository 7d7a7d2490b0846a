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

#include <utility>

#include "fa_layout.hpp"

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
// v_permlane32_swap(x, x) hands every lane both x[l % 32] and x[32 + l % 32],
// so both halves get the identical result without an LDS round trip.
__device__ __forceinline__ float halfwave_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key index (within a 32-key sub-tile) of accumulator element v of a lane in
// half-wave hh, for the 32x32 MFMA output layout.
__device__ __forceinline__ int acc_row(int v, int hh) { return (v & 3) + 8 * (v >> 2) + 4 * hh; }

// Workgroup id -> work-item id.  MI355X hands workgroups to its 8 XCDs
// round-robin (workgroup w runs on XCD w mod 8), and each XCD has its own L2.
// Work items come in groups of `gs` consecutive items that read the same K/V
// (one sequence and kv head).  Groups are dealt to the XCDs round-robin, so
// a group's items stay on one XCD and share K/V in its L2, while groups of
// different cost (packed sequences of different lengths) spread over all
// XCDs.  Groups left over after the last full round of 8 keep the identity
// order.  The map is a bijection on [0, total) when total is a multiple of gs.
__device__ __forceinline__ int xcd_remap(int w, int total, int gs) {
  const int full = (total / gs) >> 3;  // complete rounds of 8 groups
  if (w >= full * 8 * gs) return w;
  const int x = w & 7, slot = w >> 3;
  const int r = slot / gs, within = slot - r * gs;
  return (r * 8 + x) * gs + within;
}

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

// Lazy rescaling threshold, in log2 units.  The online-softmax result is exact
// for any per-row reference value r in place of the running max, as long as
// exp2(s c - r) cannot overflow: O and l are both accumulated relative to r,
// and LSE = ln2 (r + log2 l).  The reference is moved to the new maximum (and
// O, l rescaled by 2^(r_old - r_new)) only when a row's maximum exceeds it by
// more than kRescaleTau, so probabilities stay below 2^kRescaleTau and most
// tiles skip the O rescale altogether.  kRescaleTau = 0 moves it on every
// increase, which is the rescale-only-when-the-max-grows rule.
#ifndef FA_RESCALE_TAU
#define FA_RESCALE_TAU 8.0f
#endif
constexpr float kRescaleTau = FA_RESCALE_TAU;

// Largest accepted sum of one lane's probabilities of a tile formed against
// the unchanged reference (p = 2^(s c - r) <= that sum).  2^kRescaleTau
// keeps every accepted probability within the bound the row-maximum path
// gives, so both paths round the same range of values.
constexpr float kSumCap = 256.0f;
static_assert(kSumCap <= 448.0f, "accepted probabilities must stay inside the E4M3 range");

// Online-softmax probabilities for NKT score sub-tiles: new reference, the
// rescale factor alpha, probabilities (fp32 for the row sum, bf16 for the P V
// product).  Returns whether any row of the wave moved its reference.
template <int D, int NT, int NKT>
__device__ __forceinline__ bool softmax_probs(WaveState<D, NT>& st, f32x16 (&s)[NKT][NT],
                                              bf16x8 (&pb)[NKT][NT][2], float (&alpha)[NT],
                                              float c) {
  bool moved = false;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kt][t][v]);
    const float mx_c = halfwave_max(mx) * c;
    const float mref = (mx_c > st.mc[t] + kRescaleTau) ? mx_c : st.mc[t];
    moved |= mref != st.mc[t];
    // A row that has seen only masked keys keeps r = -inf; subtract 0 then so
    // that exp2(-inf - 0) = 0 instead of NaN.
    const float msub = (mref == -INFINITY) ? 0.f : mref;
    alpha[t] = fast_exp2(st.mc[t] - msub);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float pr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pr[e] = fast_exp2(fmaf(s[kt][t][8 * u + e], c, -msub));
          rs += pr[e];
        }
        pb[kt][t][u] = pack_bf16x8(pr);
      }
    st.l[t] = fmaf(alpha[t], st.l[t], rs);
    st.mc[t] = mref;
  }
  return moved;
}

template <int D, int NT>
__device__ __forceinline__ void rescale_o(WaveState<D, NT>& st, const float (&alpha)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) st.o[t][dt][v] *= alpha[t];
}

// Probabilities plus the O rescale, skipped (exactly) when no row of the wave
// moved its reference.
template <int D, int NT, int NKT>
__device__ __forceinline__ void softmax_update(WaveState<D, NT>& st, f32x16 (&s)[NKT][NT],
                                               bf16x8 (&pb)[NKT][NT][2], float c) {
  float alpha[NT];
  const bool moved = softmax_probs<D, NT, NKT>(st, s, pb, alpha, c);
  if (__any(moved)) rescale_o<D, NT>(st, alpha);
}

// ---------------------------------------------------------------------------
// Row-major K and V tiles filled straight from global memory into LDS
// (global_load_lds_dwordx4: each wave instruction writes 64 x 16 bytes of
// consecutive LDS), with the 16-byte chunks of row r XOR-swizzled by sw(r).
// gfx950's LDS has 64 banks of 4 bytes (256 bytes per clock): a 16-byte read
// serves 16 lanes per clock, an 8-byte read 32.  sw puts on distinct bank
// groups (a) the 16 consecutive rows of one K operand read (same chunk) and
// (b) the 4 rows x 4 chunks of the 32 lanes of one transposing V read.
// Rows past the end of the keys are loaded from the last valid row instead:
// their scores are masked, so they only ever meet a zero probability.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// One direct global->LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane l writes lds_dst + 16 l.  Issued as inline assembly, so that the
// compiler does not make every later LDS read wait for all such loads (it
// cannot tell the stages apart); the kernel waits for exactly the loads a
// step needs and then meets at a barrier.  M0 holds the wave's LDS
// destination; the load reads M0 one wait state after it is set.
__device__ __forceinline__ void dma16(const void* g, char* lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds_dst)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(m0) : "memory", "m0");
}

// The same load with a wave-uniform 64-bit base in SGPRs and a per-lane
// 32-bit byte offset: the address is base + offset, with no vector address
// arithmetic per load.
// lds_addr is the destination's LDS byte address (wave-uniform).
__device__ __forceinline__ void dma16_s(uint32_t off, const void* base, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(lds_addr) : "memory", "m0");
}

// The same load with the LDS destination formed as a wave-uniform scalar
// base plus a constant, so that no destination holds a scalar register of
// its own.  The add sets SCC.
template <uint32_t IMM>
__device__ __forceinline__ void dma16_si(uint32_t off, const void* base, uint32_t lds_wave) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(lds_wave), "i"(IMM) : "memory", "m0", "scc");
}

// Calls f(integral_constant<int, i>) for i = 0 .. N-1, every index a
// compile-time constant.
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// A pointer that is the same in every lane, moved to scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)p));
}

template <int D, int BC, int NW>
struct TileDMA {
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;        // rows per wave instruction
  static constexpr int NI = BC / RPI;         // wave instructions per tile
  static constexpr int PER_WAVE = NI / NW;
  static_assert(NI % NW == 0, "tile rows must split evenly over the waves");

  int off[PER_WAVE];  // element offset, from the tile's first row, of the
                      // chunk this lane fills in each of its instructions
  uint32_t obytes[PER_WAVE];  // the same in bytes (scalar-base loads)
  // The swizzle depends on the low four row bits; when consecutive
  // instructions are 16 rows apart the lane's chunk is the same in all.
  static constexpr int NCB = (RPI * NW) % 16 == 0 ? 1 : PER_WAVE;
  int row0;                // the lane's tile row in instruction 0
  uint32_t cbytes[NCB];    // byte offset of the lane's chunk in its row

  __device__ __forceinline__ static int row_of(int n, int wave, int lane) {
    return dma_row<D>(wave + n * NW, lane);
  }

  __device__ __forceinline__ void init(size_t row_stride, int wave, int lane) {
#pragma unroll
    for (int n = 0; n < PER_WAVE; ++n) {
      const int row = row_of(n, wave, lane);
      off[n] = row * (int)row_stride + (dma_chunk<D>(wave + n * NW, lane) << 3);
      obytes[n] = 2u * (uint32_t)off[n];
    }
    row0 = row_of(0, wave, lane);
#pragma unroll
    for (int n = 0; n < NCB; ++n) cbytes[n] = (uint32_t)dma_chunk<D>(wave + n * NW, lane) << 4;
  }

  // Tile rows k0..k0+BC-1 of `base` into `lds`.  Rows past klast are read
  // from row klast (their scores are masked later).
  __device__ __forceinline__ void issue(const uint16_t* __restrict__ base, size_t row_stride,
                                        int k0, int klast, char* lds, int wave, int lane) const {
    const uint16_t* tile = base + (size_t)k0 * row_stride;
    if (k0 + BC - 1 <= klast) {
#pragma unroll
      for (int n = 0; n < PER_WAVE; ++n)
        __builtin_amdgcn_global_load_lds(tile + off[n],
                                         (lds_void*)(lds + (wave + n * NW) * 1024), 16, 0, 0);
    } else {
#pragma unroll
      for (int n = 0; n < PER_WAVE; ++n) {
        const int row = row_of(n, wave, lane);
        const int src = min(k0 + row, klast);
        const uint16_t* g =
            base + (size_t)src * row_stride + (dma_chunk<D>(wave + n * NW, lane) << 3);
        __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds + (wave + n * NW) * 1024), 16, 0,
                                         0);
      }
    }
  }

  // Branch-free form of the same loads, one instruction at a time.  The
  // scalar base is the tile's first row, or row klast when the whole tile
  // lies past it; each lane's 32-bit byte offset is its row, clamped to
  // klast, times the row pitch plus its swizzled chunk.  Every address thus
  // stays inside rows 0..klast, whatever k0 is.
  struct Src {
    const uint16_t* tile;  // first row read
    int lim;               // last row of the tile that may be read, >= 0
  };
  __device__ __forceinline__ static Src src(const uint16_t* __restrict__ base, size_t row_stride,
                                            int k0, int klast) {
    const int k = min(k0, klast);
    return {base + (size_t)k * row_stride, klast - k};
  }
  // row_bytes is the row pitch in bytes (2 row_stride), below 2^24.
  template <int N>
  __device__ __forceinline__ void issue_one(const Src& s, uint32_t row_bytes, uint32_t lds_addr,
                                            int wave) const {
    static_assert(N >= 0 && N < PER_WAVE, "instruction index");
    const int r = min(row0 + N * RPI * NW, s.lim);
    dma16_s(__umul24((uint32_t)r, row_bytes) + cbytes[NCB == 1 ? 0 : N], s.tile,
            lds_addr + (wave + N * NW) * 1024);
  }

  // The same loads issued as inline assembly: the caller waits for them
  // itself (s_waitcnt vmcnt) before the barrier that precedes any read.  A
  // whole tile takes the scalar-base form (dma16_s; the byte offsets 2 off[n]
  // fit 32 bits for any tile of one sequence), a tile that runs past klast
  // the per-lane address form with its rows clamped.
  // lds_addr is the tile's LDS byte address; `lds` the same place as a pointer.
  __device__ __forceinline__ void issue_asm(const uint16_t* __restrict__ base, size_t row_stride,
                                            int k0, int klast, char* lds, uint32_t lds_addr,
                                            int wave, int lane) const {
    const uint16_t* tile = base + (size_t)k0 * row_stride;
    if (k0 + BC - 1 <= klast) {
#pragma unroll
      for (int n = 0; n < PER_WAVE; ++n)
        dma16_s(obytes[n], tile, lds_addr + (wave + n * NW) * 1024);
    } else {
#pragma unroll
      for (int n = 0; n < PER_WAVE; ++n) {
        const int row = row_of(n, wave, lane);
        const int src = min(k0 + row, klast);
        const uint16_t* g =
            base + (size_t)src * row_stride + (dma_chunk<D>(wave + n * NW, lane) << 3);
        dma16(g, lds + (wave + n * NW) * 1024);
      }
    }
  }
};

// Per-lane LDS byte offsets of the MFMA operand reads from swizzled K / V
// tiles: one base register per head-dim step plus compile-time offsets for
// the key sub-tile (the swizzle depends only on the low row bits, which the
// lane fixes).
template <int D>
struct LdsRead {
  static constexpr int KS = D / 16;  // score k-steps
  static constexpr int DT = D / 32;  // head-dim blocks of the P V product
  uint32_t kb[KS];                   // K operand of score k-step st, keys 0..31
  uint32_t vb[DT][2];                // V operand of block dt, key rows +0 / +8

  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int st = 0; st < KS; ++st) kb[st] = k_read_offset<D>(lane, st);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) vb[dt][sec] = v_read_offset<D>(lane, dt, sec);
  }

  // A operand of S^T = K Q^T: keys kt*32.., head-dim step st.  Key rows
  // kt*32 + m32 share the swizzle of m32.
  __device__ __forceinline__ bf16x8 k(const char* __restrict__ lds, int kt, int st) const {
    return *reinterpret_cast<const bf16x8*>(lds + kb[st] + kt * 64 * D);
  }

  // A operand of O^T = V^T P^T for head-dim rows dt*32.. and the 8 keys of
  // the lane's half-wave in the 16-key step (kt, u), from a row-major V tile,
  // with two transposing LDS reads.  ds_read_b64_tr_b16 transposes within
  // each group of 16 lanes: result lane i, element j is element i & 3 of the
  // 8 bytes addressed by source lane 4 j + (i >> 2).  Rows kt*32 + 16 u + r
  // share the swizzle of r.
  __device__ __forceinline__ bf16x8 v(const char* __restrict__ lds, int kt, int u, int dt) const {
    const char* a = lds + (kt * 32 + 16 * u) * 2 * D;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(a + vb[dt][0]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(a + vb[dt][1]));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
  }
};

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Waits for every outstanding vector-memory access through the builtin,
// whose effect the compiler's wait-count tracking sees (it does not see an
// asm wait).  Loads the compiler issued before this point (the Q fragments)
// are then known complete, so it places no waits for them further on.  Such
// waits would otherwise land inside the key loop, where the hardware counter
// also counts the asm-issued tile loads, and stall each step on loads issued
// a few instructions earlier.
__device__ __forceinline__ void vm_drain() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt not waited on
}


// S^T sub-tiles kt = 0..NKT-1 (keys kt*32..) of a swizzled K tile, with the
// independent accumulators interleaved so consecutive MFMAs do not depend on
// each other; the fragments of step st+1 are read while step st's MFMAs run.
template <int D, int NT, int NKT, bool PREFETCH = true>
__device__ __forceinline__ void scores_tile(f32x16 (&s)[NKT][NT], const char* __restrict__ k_lds,
                                            const LdsRead<D>& rd,
                                            const bf16x8 (&qf)[NT][D / 16]) {
  bf16x8 a[2][NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) a[0][kt] = rd.k(k_lds, kt, 0);
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (!PREFETCH && st > 0) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) a[st & 1][kt] = rd.k(k_lds, kt, st);
    }
    if (PREFETCH && st + 1 < D / 16) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) a[(st + 1) & 1][kt] = rd.k(k_lds, kt, st + 1);
    }
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        s[kt][t] = mfma_32x32x16(a[st & 1][kt], qf[t][st], st == 0 ? f32x16{} : s[kt][t]);
  }
}

// O^T += V^T P^T over NKT 32-key sub-tiles; the D/32 accumulators of a step
// are independent and interleaved.
template <int D, int NT, int NKT>
__device__ __forceinline__ void pv_tile(WaveState<D, NT>& st, const char* __restrict__ v_lds,
                                        const LdsRead<D>& rd, const bf16x8 (&pb)[NKT][NT][2]) {
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16x8 a = rd.v(v_lds, kt, u, dt);
#pragma unroll
        for (int t = 0; t < NT; ++t) st.o[t][dt] = mfma_32x32x16(a, pb[kt][t][u], st.o[t][dt]);
      }
}

// Stores a wave's 32 rows x D accumulator times `scale` as bf16 or fp32 rows:
// row r of the wave goes to out + r * row_pitch (bytes), for r < rows.  Lane
// (m32, hh) holds row m32, values dt*32 + 8g + 4hh + 0..3 in registers
// 4g .. 4g+3 of acc[dt] (the 32x32 MFMA output layout of O^T-style products).
// The rows pass through `stg`, this wave's LDS area (32 x 256 bytes; only
// 32 x 128 for bf16 at D = 64), in pieces of 32 rows x up to 256 bytes, so
// that every global store writes whole 16-byte chunks of a contiguous run of
// a row: stores straight from the accumulator layout write 8 bytes per lane,
// and lines filled by several partial writes cost more.  Row r of a piece
// holds its chunks XOR-swizzled by r.  The stores are non-temporal: callers
// write outputs that the same launch does not read.
template <int D>
__device__ __forceinline__ void store_rows_lds(const f32x16 (&acc)[D / 32], float scale,
                                               char* out, size_t row_pitch, int rows, bool f32,
                                               char* stg, int lane) {
  static_assert(D == 64 || D == 128, "head dim");
  const int m32 = lane & 31, hh = lane >> 5;
  // piece pc of every row: lanes of one row take its 16-byte chunks
  auto piece_out = [&](auto pw_c, const int pc) __attribute__((always_inline)) {
    constexpr int PW = decltype(pw_c)::value;  // bytes of a row per piece
    constexpr int LPR = PW / 16;               // lanes (chunks) per row
    constexpr int RPI = 64 / LPR;              // rows per instruction
    constexpr int NI = 32 / RPI;
    const int c = lane % LPR, r0 = lane / LPR;
    u32x4 w[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = RPI * i + r0;
      w[i] = *reinterpret_cast<const u32x4*>(stg + r * PW + ((c ^ (r & (LPR - 1))) << 4));
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = RPI * i + r0;
      if (r < rows)
        __builtin_nontemporal_store(
            w[i], reinterpret_cast<u32x4*>(out + (size_t)r * row_pitch + PW * pc + 16 * c));
    }
  };
  if (f32) {
    // 4D bytes a row: pieces of 256 bytes hold head-dim blocks dt = 2 pc, 2 pc + 1
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = (dt & 1) * 8 + 2 * g + hh;
        const f32x4 w = {acc[dt][4 * g] * scale, acc[dt][4 * g + 1] * scale,
                         acc[dt][4 * g + 2] * scale, acc[dt][4 * g + 3] * scale};
        *reinterpret_cast<f32x4*>(stg + m32 * 256 + ((ch ^ (m32 & 15)) << 4)) = w;
      }
      if (dt & 1) piece_out(std::integral_constant<int, 256>{}, dt >> 1);
    }
  } else {
    // 2D bytes a row, one piece: chunk 4 dt + g, half hh
    constexpr int PW = 2 * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = dt * 4 + g;
        const u32x2 w = {pack_bf16x2(acc[dt][4 * g] * scale, acc[dt][4 * g + 1] * scale),
                         pack_bf16x2(acc[dt][4 * g + 2] * scale, acc[dt][4 * g + 3] * scale)};
        *reinterpret_cast<u32x2*>(stg + m32 * PW + ((ch ^ (m32 & (PW / 16 - 1))) << 4) +
                                  8 * hh) = w;
      }
    piece_out(std::integral_constant<int, PW>{}, 0);
  }
}

}  // namespace fa
