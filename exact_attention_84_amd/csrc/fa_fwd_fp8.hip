// FP8 attention forward: both matrix products on gfx950's FP8 matrix cores
// (the FlashAttention 3 low-precision item of "推理优化 | FlashAttention 1-4
// 详解", section FlashAttention 3 的硬件特性利用: the forward's products in
// FP8, the backward in BF16).  Q, K and V arrive as OCP E4M3 codes with one
// fp32 descale per tensor (real value = descale * code value); the result is
// attention of the real tensors, with O in bf16 or fp32 and the natural-log
// LSE in fp32.
//
// Same decomposition as the bf16 forward (a workgroup per query tile of BR =
// 32 NW rows of one (sequence, query head), causal tiles paired heavy with
// light, Q in registers, K/V tiles of 64 keys streamed into LDS by direct
// loads, online softmax in base 2 with a lazy reference), with the FP8 data
// path:
//   * S^T = K Q^T with v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales):
//     2 k-steps of 64 head-dim values per 32-key sub-tile;
//   * the descales fold into the softmax constant c = scale dq dk log2 e, and
//     dv multiplies O at the end;
//   * P = exp2(s c - r) <= 2^8 (the lazy reference stays within 8 of the row
//     maximum) is rounded to E4M3 (v_cvt_pk_fp8_f32, nearest-even; 256 < 448
//     never saturates) straight from the accumulators into the B operand of
//     O^T = V^T P^T; the row sum l adds the unrounded values;
//   * V^T comes from the row-major V tile with transposing byte reads
//     (ds_read_b64_tr_b8), one MFMA of 64 keys per 32 head-dim rows.
// The LDS layouts, and which key each operand slot holds, are those of
// fa_layout.hpp (k8_*, v8_*, pv8_key).
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kD8 = 128;              // head dim
constexpr int kBC8 = 64;              // keys per tile
constexpr int kTile8 = kBC8 * kD8;    // bytes per K or V tile

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Direct global->LDS fill of one 64-row FP8 tile: 8 wave instructions of
// 64 x 16 bytes, NW waves issuing 8 / NW each.  Rows past klast are read from
// row klast (their scores are masked, so they only meet zero probabilities).
template <int NW, bool V_TILE>
struct Dma8 {
  static constexpr int PER_WAVE = 8 / NW;
  static_assert(8 % NW == 0, "tile instructions must split evenly over the waves");
  int row[PER_WAVE];         // the lane's tile row in each instruction
  uint32_t cbytes[PER_WAVE];  // byte offset of its 16-byte chunk in that row

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int n = 0; n < PER_WAVE; ++n) {
      const int inst = wave + n * NW;
      row[n] = dma8_row(inst, lane);
      cbytes[n] = (uint32_t)dma8_chunk(inst, lane, V_TILE) << 4;
    }
  }
  // With no branch: the scalar base is the tile's first row (row klast when
  // the whole tile lies past it) and each lane's 32-bit offset is its row,
  // clamped to klast, times the pitch plus its chunk, so every address stays
  // inside rows 0..klast.  row_stride is below 2^24.
  __device__ __forceinline__ void issue(const uint8_t* __restrict__ base, int row_stride, int k0,
                                        int klast, char* lds, int wave) const {
    const int k = min(k0, klast);
    const uint8_t* tile = base + (size_t)k * row_stride;
    const int lim = klast - k;
    const uint32_t at = lds_address(lds);
#pragma unroll
    for (int n = 0; n < PER_WAVE; ++n) {
      const uint32_t r = (uint32_t)min(row[n], lim);
      dma16_s(__umul24(r, (uint32_t)row_stride) + cbytes[n], tile,
              at + (wave + n * NW) * 1024);
    }
  }
};

// Per-lane LDS offsets of the operand reads.
struct Rd8 {
  uint32_t kb[2][2];  // K: [k-step][16-byte half], key rows 0..31
  uint32_t vb[4];     // V^T: [head-dim block], read q = 0

  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int u = 0; u < 2; ++u) kb[st][u] = k8_read_offset(lane, st, u);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) vb[dt] = v8_read_offset(lane, dt);
  }
  // A operand of S^T = K Q^T: keys 32 kt.., head-dim 64 st + 32 hh ..
  __device__ __forceinline__ i32x8 k(const char* __restrict__ lds, int kt, int st) const {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(lds + kb[st][0] + kt * 32 * kD8);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(lds + kb[st][1] + kt * 32 * kD8);
    const i32x8 r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    return r;
  }
  // A operand of O^T = V^T P^T for head-dim rows 32 dt..: four transposing
  // reads, read q filling slots 8 q .. 8 q + 7.
  __device__ __forceinline__ i32x8 v(const char* __restrict__ lds, int dt) const {
    i32x8 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) i32x2*)(lds + vb[dt] + 2048 * q));
      r[2 * q] = w[0];
      r[2 * q + 1] = w[1];
    }
    return r;
  }
};

// Waits until at most `tiles` tile loads of this wave (PER instructions
// each) are still in flight: the loads of a step complete in issue order.
template <int PER>
__device__ __forceinline__ void wait_tiles_upto(int tiles) {
  if (tiles <= 0)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (tiles == 1)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory");
}

struct State8 {
  i32x8 qf[2];     // Q^T, B operand of S^T = K Q^T, per k-step
  f32x16 o[4];     // O^T accumulators (unnormalised), per 32 head-dim rows
  float mc;        // reference, in units of c (log2)
  float l;         // row sum of this half-wave's keys, relative to mc
};

// Online-softmax step for one 64-key tile: new reference, rescale factor,
// probabilities rounded to E4M3 into the B operand (slot 16 kt + v holds
// element v of sub-tile kt).  Returns whether the row moved its reference.
__device__ __forceinline__ bool softmax8(State8& st, f32x16 (&s)[2], i32x8& pb, float& alpha,
                                         float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kt][v]);
  const float mx_c = halfwave_max(mx) * c;
  const float mref = (mx_c > st.mc + kRescaleTau) ? mx_c : st.mc;
  const bool moved = mref != st.mc;
  // a row that has seen only masked keys keeps -inf; subtract 0 then
  const float msub = (mref == -INFINITY) ? 0.f : mref;
  alpha = fast_exp2(st.mc - msub);
  float rs = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = 4 * w + e;
      pr[e] = fast_exp2(fmaf(s[idx >> 4][idx & 15], c, -msub));
      rs += pr[e];
    }
    // the first conversion keeps the high half of its third operand, which
    // the second overwrites: any register will do, and a dead one saves the
    // compiler zeroing a fresh one
    int x =
        __builtin_amdgcn_cvt_pk_fp8_f32(pr[0], pr[1], __builtin_bit_cast(int, pr[1]), false);
    x = __builtin_amdgcn_cvt_pk_fp8_f32(pr[2], pr[3], x, true);
    pb[w] = x;
  }
  st.l = fmaf(alpha, st.l, rs);
  st.mc = mref;
  return moved;
}

// Sets to -inf every score of a 64-key tile past the lane's limit: element v
// of sub-tile kt holds key (v & 3) + 8 (v >> 2) + 32 kt + 4 hh of the tile,
// and lim already has 4 hh taken off.
__device__ __forceinline__ void mask8(f32x16 (&s)[2], int lim) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if ((v & 3) + 8 * (v >> 2) + 32 * kt > lim) s[kt][v] = -INFINITY;
}

// S^T sub-tiles of a 64-key tile: two k-steps of 64 head-dim values each.
__device__ __forceinline__ void scores8(f32x16 (&s)[2], const char* __restrict__ k_cur,
                                        const Rd8& rd, const State8& st) {
  const i32x8 a0 = rd.k(k_cur, 0, 0), a1 = rd.k(k_cur, 1, 0);
  const i32x8 b0 = rd.k(k_cur, 0, 1), b1 = rd.k(k_cur, 1, 1);
  s[0] = mfma_fp8(a0, st.qf[0], f32x16{});
  s[1] = mfma_fp8(a1, st.qf[0], f32x16{});
  s[0] = mfma_fp8(b0, st.qf[1], s[0]);
  s[1] = mfma_fp8(b1, st.qf[1], s[1]);
}

// One steady step: S_j = K_j Q^T, then the four P_{j-1} V_{j-1} MFMAs, each
// followed by the exponentials of 8 of the lane's keys (sched_barrier fences
// keep that order), so that the ALUs work while the matrix core runs.  The
// probabilities are formed against the row's current reference r with no
// row maximum; every p is at most the lane's sum of them, so when no sum
// exceeds kSumCap (and none is inf or NaN) the reference stays and alpha = 1.
// Otherwise the scores, kept unchanged, go through softmax8, which moves the
// references.  pout receives P_j; returns whether the row moved its reference
// (alpha then holds the rescale factor, applied before P_j V_j).
__device__ __forceinline__ bool steady8(State8& st, const char* __restrict__ k_cur,
                                        const char* __restrict__ v_prev, const Rd8& rd,
                                        const i32x8& pin, i32x8& pout, float& alpha, float c,
                                        bool masked, int lim) {
  f32x16 s[2];
  scores8(s, k_cur, rd, st);
  if (masked) mask8(s, lim);
  float rs = 0.f;
  i32x8 pk;
  i32x8 va = rd.v(v_prev, 0);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const i32x8 vcur = va;
    if (dt < 3) va = rd.v(v_prev, dt + 1);
    st.o[dt] = mfma_fp8(vcur, pin, st.o[dt]);
    // keep the product in this slice: without a use here the compiler sinks
    // the four products past the accept branch below, and the exponentials
    // then run with the matrix core idle (the asm emits no instruction)
    asm volatile("" ::"v"(st.o[dt]));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int w = 2 * dt; w < 2 * dt + 2; ++w) {
      float pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = 4 * w + e;
        pr[e] = fast_exp2(fmaf(s[idx >> 4][idx & 15], c, -st.mc));
        rs += pr[e];
      }
      // (as in softmax8: the third operand only fills the half that the
      // second conversion overwrites)
      int x =
          __builtin_amdgcn_cvt_pk_fp8_f32(pr[0], pr[1], __builtin_bit_cast(int, pr[1]), false);
      x = __builtin_amdgcn_cvt_pk_fp8_f32(pr[2], pr[3], x, true);
      pk[w] = x;
      // keep the conversion in this slice
      asm volatile("" ::"v"(x));
    }
    asm volatile("" : "+v"(rs));
    __builtin_amdgcn_sched_barrier(0);
  }
  if (__builtin_expect(__all(rs <= kSumCap), 1)) {
    pout = pk;
    st.l += rs;
    alpha = 1.f;
    return false;
  }
  // the row outgrew its reference (or has none yet): the row-maximum path
  // on the unchanged scores
  return softmax8(st, s, pout, alpha, c);
}

}  // namespace

template <int NW, bool CAUSAL, bool PAIR>
__device__ __forceinline__ void fwd_fp8_body(const FwdParams& p, float v_descale) {
  constexpr int BR = NW * 32;
  // Three stages of K and V: tiles j+1 and j+2 stream in while tile j is used.
  __shared__ __attribute__((aligned(1024))) char k_lds[3 * kTile8];
  __shared__ __attribute__((aligned(1024))) char v_lds[3 * kTile8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m32 = lane & 31, hh = lane >> 5;

  const int item = xcd_remap(blockIdx.x, p.total, p.group * p.n_items);
  const int it = item % p.n_items;
  int rest = item / p.n_items;
  const int hg = rest % p.group;
  rest /= p.group;
  const int kvh = rest % p.hkv;
  const int b = rest / p.hkv;
  const int h = kvh * p.group + hg;

  int q_start, Lq, k_start, Lk;
  if (p.cu_q) {
    q_start = p.cu_q[b];
    Lq = p.cu_q[b + 1] - q_start;
    k_start = p.cu_k[b];
    Lk = p.cu_k[b + 1] - k_start;
  } else {
    q_start = b * p.seqlen_q;
    Lq = p.seqlen_q;
    k_start = b * p.seqlen_k;
    Lk = p.seqlen_k;
  }
  const uint8_t* q8 = reinterpret_cast<const uint8_t*>(p.q);
  const uint8_t* k8 = reinterpret_cast<const uint8_t*>(p.k);
  const uint8_t* v8 = reinterpret_cast<const uint8_t*>(p.v);
  const int q_stride = p.hq * kD8;   // bytes per token row
  const int kv_stride = p.hkv * kD8;
  const uint8_t* kbase = k8 + (size_t)k_start * kv_stride + (size_t)kvh * kD8;
  const uint8_t* vbase = v8 + (size_t)k_start * kv_stride + (size_t)kvh * kD8;

  auto run_tile = [&](const int qt) __attribute__((always_inline)) {
    const int q0 = qt * BR;
    const int delta = Lk - Lq;  // bottom-right causal offset
    int n_kt = (Lk + kBC8 - 1) / kBC8;
    if (CAUSAL) {
      const int last_key = min(Lk - 1, q0 + BR - 1 + delta);
      n_kt = last_key < 0 ? 0 : min(n_kt, last_key / kBC8 + 1);
    }
    const int qw0 = q0 + wave * 32;
    const bool wave_active = qw0 < Lq;
    const int wave_last_key = CAUSAL ? min(Lk - 1, qw0 + 31 + delta) : Lk - 1;
    const int wn =
        (wave_active && wave_last_key >= 0) ? min(n_kt, wave_last_key / kBC8 + 1) : 0;

    Dma8<NW, false> dk;
    Dma8<NW, true> dv;
    dk.init(wave, lane);
    dv.init(wave, lane);
    Rd8 rd;
    rd.init(lane);
    // K_0, then K_1 and V_0 (step j waits for K_j and V_{j-1}, issued a step
    // before the loads it may leave in flight)
    if (n_kt > 0) dk.issue(kbase, kv_stride, 0, Lk - 1, k_lds, wave);
    if (n_kt > 1) dk.issue(kbase, kv_stride, kBC8, Lk - 1, k_lds + kTile8, wave);
    if (n_kt > 0) dv.issue(vbase, kv_stride, 0, Lk - 1, v_lds, wave);

    State8 st;
    st.mc = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) st.o[dt][v] = 0.f;
    const int qi = qw0 + m32;
    {
      const uint8_t* qp = q8 + (size_t)(q_start + qi) * q_stride + (size_t)h * kD8 + 32 * hh;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
        if (qi < Lq) {
          lo = *reinterpret_cast<const u32x4*>(qp + 64 * s);
          hi = *reinterpret_cast<const u32x4*>(qp + 64 * s + 16);
        }
        const i32x8 r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        st.qf[s] = r;
      }
      // Q has landed before the key loop: otherwise the compiler's wait for
      // it sits at its first use inside the loop and waits for every tile
      // load in flight on each step
      asm volatile("" ::"v"(st.qf[0]), "v"(st.qf[1]));
    }
    // last admissible key of this lane's row minus 4 hh (the lane's key
    // offset inside a 32-key sub-tile); tile j masks against lim - 64 j
    const int row_lim = (CAUSAL ? min(Lk - 1, qi + delta) : Lk - 1) - 4 * hh;
    auto edge_tile = [&](int j) {
      const int k0 = j * kBC8;
      return (k0 + kBC8 > Lk) || (CAUSAL && k0 + kBC8 - 1 > qw0 + delta);
    };

    i32x8 p_a, p_b;
    float alpha = 1.f;
    bool moved = false;
    constexpr int PER = Dma8<NW, false>::PER_WAVE;
    int s0 = 0;  // stage of K_j and V_j: j mod 3
    // Step j: K_j and V_{j-1} have landed once at most the previous step's
    // loads (K_{j+1}, V_j) are in flight; then K_{j+2} and V_{j+1} stream
    // into the stages that K_{j-1} and V_{j-2} used.  Sets the stages of K_j
    // and V_{j-1}.
    const char* k_cur;
    const char* v_prev;
    auto stage = [&](int j) {
      const int s1 = s0 == 2 ? 0 : s0 + 1;  // (j + 1) mod 3
      const int s2 = s1 == 2 ? 0 : s1 + 1;  // (j + 2) mod 3 = (j - 1) mod 3
      wait_tiles_upto<PER>((j + 1 < n_kt ? 1 : 0) + (j < n_kt ? 1 : 0));
      __syncthreads();
      if (j + 2 < n_kt)
        dk.issue(kbase, kv_stride, (j + 2) * kBC8, Lk - 1, k_lds + s2 * kTile8, wave);
      if (j + 1 < n_kt)
        dv.issue(vbase, kv_stride, (j + 1) * kBC8, Lk - 1, v_lds + s1 * kTile8, wave);
      k_cur = k_lds + s0 * kTile8;
      v_prev = v_lds + s2 * kTile8;
      s0 = s1;
    };
    // the O rescale of step j-1's softmax lands between P_{j-2} V and P_{j-1} V
    auto rescale = [&]() {
      if (__any(moved)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) st.o[dt][v] *= alpha;
      }
    };
    // One step done phase by phase: the first tile (no P V yet), the final
    // P V, and steps where this wave has nothing left.  P_{j-1} is in p_a.
    auto general_step = [&](int j) {
      stage(j);
      if (j >= 1 && j <= wn) {
        rescale();
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) st.o[dt] = mfma_fp8(rd.v(v_prev, dt), p_a, st.o[dt]);
      }
      if (j < wn) {
        f32x16 s[2];
        scores8(s, k_cur, rd, st);
        if (edge_tile(j)) mask8(s, row_lim - j * kBC8);
        moved = softmax8(st, s, p_a, alpha, p.c);
      }
    };
    auto steady = [&](int j, const i32x8& pin, i32x8& pout) {
      stage(j);
      rescale();
      moved = steady8(st, k_cur, v_prev, rd, pin, pout, alpha, p.c, edge_tile(j),
                      row_lim - j * kBC8);
    };
    // The same step with its stage S0 = j mod 3 known at compile time, so
    // that the stage offsets of the operand reads are instruction immediates
    // instead of a vector add per read base (8 a step).
    auto steady_s = [&](auto s0c, int j, const i32x8& pin, i32x8& pout)
        __attribute__((always_inline)) {
      constexpr int S0 = decltype(s0c)::value;
      constexpr int S1 = (S0 + 1) % 3, S2 = (S0 + 2) % 3;
      wait_tiles_upto<PER>((j + 1 < n_kt ? 1 : 0) + (j < n_kt ? 1 : 0));
      __syncthreads();
      if (j + 2 < n_kt)
        dk.issue(kbase, kv_stride, (j + 2) * kBC8, Lk - 1, k_lds + S2 * kTile8, wave);
      if (j + 1 < n_kt)
        dv.issue(vbase, kv_stride, (j + 1) * kBC8, Lk - 1, v_lds + S1 * kTile8, wave);
      rescale();
      moved = steady8(st, k_lds + S0 * kTile8, v_lds + S2 * kTile8, rd, pin, pout, alpha, p.c,
                      edge_tile(j), row_lim - j * kBC8);
    };
    int j = 0;
    if (wn > 1) {
      general_step(0);
      j = 1;
      // unrolled by six: the stage (j mod 3) and the probability registers
      // (j mod 2) are both static; step j = 1 uses stage 1 (the generic step
      // 0 used stage 0)
      using C0 = std::integral_constant<int, 0>;
      using C1 = std::integral_constant<int, 1>;
      using C2 = std::integral_constant<int, 2>;
#pragma clang loop unroll(disable)
      while (j + 5 < wn) {
        steady_s(C1{}, j, p_a, p_b);
        steady_s(C2{}, j + 1, p_b, p_a);
        steady_s(C0{}, j + 2, p_a, p_b);
        steady_s(C1{}, j + 3, p_b, p_a);
        steady_s(C2{}, j + 4, p_a, p_b);
        steady_s(C0{}, j + 5, p_b, p_a);
        j += 6;
      }
      s0 = j % 3;  // the run-time stage of the steps that follow
      // the rest unrolled by two so that the probability registers swap
      // statically; no exit between the two halves, which would make the
      // compiler copy the new probabilities at every step for the exit's sake
#pragma clang loop unroll(disable)
      while (j + 1 < wn) {
        steady(j, p_a, p_b);
        steady(j + 1, p_b, p_a);
        j += 2;
      }
      if (j < wn) {
        steady(j, p_a, p_b);
        p_a = p_b;  // the generic step expects P_{j-1} in p_a
        ++j;
      }
    }
#pragma clang loop unroll(disable)
    for (; j <= n_kt; ++j) general_step(j);

    // ---- epilogue: O dv / l, LSE = ln 2 (r + log2 l) ----
    const float lt = halfwave_sum(st.l);
    const float inv = lt > 0.f ? v_descale / lt : 0.f;
    const float lse = lt > 0.f ? (st.mc + __log2f(lt)) * kLn2 : -INFINITY;
    if (qi < Lq && hh == 0) p.lse[(size_t)(q_start + qi) * p.hq + h] = lse;
    // O goes out through 8 KB of the K/V stages, free once every wave is past
    // its last P V, as whole 16-byte chunks of contiguous row runs
    __syncthreads();
    const size_t esz = p.o_f32 ? 4 : 2;
    store_rows_lds<kD8>(st.o, inv,
                        reinterpret_cast<char*>(p.o) +
                            ((size_t)(q_start + qw0) * p.hq + h) * kD8 * esz,
                        (size_t)p.hq * kD8 * esz, Lq - qw0, p.o_f32 != 0,
                        wave < 3 ? k_lds + wave * kTile8 : v_lds, lane);
  };  // run_tile

  if constexpr (PAIR) {
    // causal: tile n-1-i (heaviest) with tile i, per sequence
    const int first = (Lq + BR - 1) / BR - 1 - it;
    if (first < it) return;  // past the middle of a shorter sequence (uniform)
    run_tile(first);
    if (it < first) {
      __syncthreads();  // every wave is done with the first tile's LDS stages
      run_tile(it);
    }
  } else {
    if (it * BR < Lq) run_tile(it);
  }
}

template <int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_fp8_kernel(const FwdParams p, float v_descale) {
  fwd_fp8_body<NW, CAUSAL, CAUSAL>(p, v_descale);
}

template __global__ void fwd_fp8_kernel<4, false>(const FwdParams, float);
template __global__ void fwd_fp8_kernel<4, true>(const FwdParams, float);

hipError_t launch_fwd_fp8(const FwdParams& p, bool causal, float v_descale, hipStream_t stream) {
  auto go = [&](auto kern, int threads) {
    hipLaunchKernelGGL(kern, dim3(p.total), dim3(threads), 0, stream, p, v_descale);
    return hipGetLastError();
  };
  if (p.waves != 4) return hipErrorInvalidValue;
  return causal ? go(fwd_fp8_kernel<4, true>, 256) : go(fwd_fp8_kernel<4, false>, 256);
}

}  // namespace fa
