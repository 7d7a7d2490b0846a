// Fused attention forward at head dim 128 with 64 query rows per wavefront
// (fixed-length batches and packed sequences, causal or not, MHA or GQA).
//
// The method is the one of fa_fwd.hip ("FlashAttention — IO 感知的精确注意力
// kernel", section 2.3 step 4: the Q tile stays on chip while K/V tiles stream
// through; "推理优化 | FlashAttention 1-4 详解", section Online Softmax 数学推导:
// running max, running sum, rescaled output, one division at the end).  What
// changes is how one wavefront maps onto gfx950:
//
// * A wave owns 64 query rows (two groups of 32).  Every K and V operand it
//   reads from LDS feeds two matrix instructions, one per row group, so the
//   LDS bytes per flop are half those of a 32-row wave.  The same page's
//   FlashAttention 2 notes name fewer shared-memory reads per flop as the
//   lever (section FlashAttention 2 的工程优化).
// * O for 64 rows x 128 head-dim values is 128 fp32 registers per lane.  It
//   lives in the accumulation registers a0..a127 for the whole tile and is
//   touched only by the inline assembly below: the P V products accumulate
//   into it in place, the rare rescale reads and writes it, and the epilogue
//   reads it once.  No compiler-visible value ever occupies an AGPR (the
//   score products are built in VGPR form), so nothing else can move or
//   overwrite it.  One wave runs per SIMD (about 180 VGPRs + 128 AGPRs).
// * The key loop is pipelined three deep within the wave: sub-step j issues
//   the score products of key block j+1 and the P V products of block j-1,
//   32 matrix instructions that do not depend on the softmax of block j,
//   and interleaves that softmax's exponentials with them.  All of a step's
//   ALU work thus overlaps its matrix work ("推理优化 | FlashAttention 1-4
//   详解", section FlashAttention 3 的硬件特性利用: overlap of GEMM and
//   softmax, done here inside one wavefront).
//
// Keys move in sub-steps of 32 (one 32x32 score block per row group) and
// LDS stages of 64 (one barrier per two sub-steps).
#include <atomic>
#include <utility>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace wide {

constexpr int D = 128;
constexpr int NT = 2;                    // 32-row groups per wave
constexpr int SUB = 32;                  // keys per pipeline sub-step
constexpr int STG = 64;                  // keys per LDS stage
constexpr int STG_BYTES = STG * D * 2;   // 16 KB
constexpr int kEpiBytes = 32 * 256;      // a wave's epilogue area: 32 rows x 256 bytes

// ---------------------------------------------------------------------------
// O^T accumulators in hard-named AGPRs: block b = 4 t + dt (row group t,
// head-dim rows 32 dt..32 dt+31) is a[16 b .. 16 b + 15], in the 32x32 MFMA
// output layout (lane l: query column l % 32, head-dim rows
// (v & 3) + 8 (v >> 2) + 4 (l >> 5) for register v).
//
// Inline assembly is not covered by the compiler's hazard checks, so these
// helpers carry their own waits:
//   * a matrix instruction reading a VGPR that a vector instruction wrote in
//     the two preceding cycles needs 2 wait states; the callers feed P and V
//     operands produced at least a slice earlier (checked on the generated
//     code by tests/test_fwd_wide_isa.py);
//   * reading an accumulator written by an in-flight matrix instruction needs
//     the instruction's passes plus a few states: 32 (two s_nop 15) before
//     the rescale and the epilogue read;
//   * an accumulator written by v_accvgpr_write and then read as srcC needs
//     2 states: s_nop 2 after the writes.
// ---------------------------------------------------------------------------
#define FA_ACC_CLOBBER_0 "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15"
#define FA_ACC_CLOBBER_1 "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31"
#define FA_ACC_CLOBBER_2 "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47"
#define FA_ACC_CLOBBER_3 "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63"
#define FA_ACC_CLOBBER_4 "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79"
#define FA_ACC_CLOBBER_5 "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95"
#define FA_ACC_CLOBBER_6 "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111"
#define FA_ACC_CLOBBER_7 "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127"

template <int B>
struct Acc;

#define FA_ACC_RANGE(B) "a[16*" #B ":16*" #B "+15]"
#define FA_DEFINE_ACC(B)                                                                        \
  template <>                                                                                   \
  struct Acc<B> {                                                                               \
    /* O^T block += A * B (A = V^T fragment, B = P^T fragment) */                               \
    static __device__ __forceinline__ void mfma(bf16x8 a, bf16x8 b) {                           \
      asm volatile("v_mfma_f32_32x32x16_bf16 " FA_ACC_RANGE(B) ", %0, %1, " FA_ACC_RANGE(B)    \
                   :: "v"(a), "v"(b) : FA_ACC_CLOBBER_##B);                                     \
    }                                                                                           \
    static __device__ __forceinline__ void zero() {                                             \
      asm volatile(".irp r, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15\n\t"                          \
                   "v_accvgpr_write_b32 a[16*" #B "+\\r], 0\n\t.endr" ::: FA_ACC_CLOBBER_##B);  \
    }                                                                                           \
    /* block *= alpha, four registers at a time; the caller has waited for */                   \
    /* the matrix instructions that wrote the block */                                         \
    static __device__ __forceinline__ void scale(float alpha) {                                 \
      float t0, t1, t2, t3;                                                                     \
      asm volatile(".irp r, 0,4,8,12\n\t"                                                       \
                   "v_accvgpr_read_b32 %0, a[16*" #B "+\\r]\n\t"                                \
                   "v_accvgpr_read_b32 %1, a[16*" #B "+\\r+1]\n\t"                              \
                   "v_accvgpr_read_b32 %2, a[16*" #B "+\\r+2]\n\t"                              \
                   "v_accvgpr_read_b32 %3, a[16*" #B "+\\r+3]\n\t"                              \
                   "v_mul_f32 %0, %4, %0\n\t"                                                   \
                   "v_mul_f32 %1, %4, %1\n\t"                                                   \
                   "v_mul_f32 %2, %4, %2\n\t"                                                   \
                   "v_mul_f32 %3, %4, %3\n\t"                                                   \
                   "v_accvgpr_write_b32 a[16*" #B "+\\r], %0\n\t"                               \
                   "v_accvgpr_write_b32 a[16*" #B "+\\r+1], %1\n\t"                             \
                   "v_accvgpr_write_b32 a[16*" #B "+\\r+2], %2\n\t"                             \
                   "v_accvgpr_write_b32 a[16*" #B "+\\r+3], %3\n\t"                             \
                   ".endr"                                                                      \
                   : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)                                 \
                   : "v"(alpha)                                                                 \
                   : FA_ACC_CLOBBER_##B);                                                       \
    }                                                                                           \
    /* the 16 values of the block; the caller has waited for the writers */                    \
    static __device__ __forceinline__ void read(float (&x)[16]) {                               \
      asm volatile("v_accvgpr_read_b32 %0, a[16*" #B "+0]\n\t"                                  \
                   "v_accvgpr_read_b32 %1, a[16*" #B "+1]\n\t"                                  \
                   "v_accvgpr_read_b32 %2, a[16*" #B "+2]\n\t"                                  \
                   "v_accvgpr_read_b32 %3, a[16*" #B "+3]\n\t"                                  \
                   "v_accvgpr_read_b32 %4, a[16*" #B "+4]\n\t"                                  \
                   "v_accvgpr_read_b32 %5, a[16*" #B "+5]\n\t"                                  \
                   "v_accvgpr_read_b32 %6, a[16*" #B "+6]\n\t"                                  \
                   "v_accvgpr_read_b32 %7, a[16*" #B "+7]\n\t"                                  \
                   "v_accvgpr_read_b32 %8, a[16*" #B "+8]\n\t"                                  \
                   "v_accvgpr_read_b32 %9, a[16*" #B "+9]\n\t"                                  \
                   "v_accvgpr_read_b32 %10, a[16*" #B "+10]\n\t"                                \
                   "v_accvgpr_read_b32 %11, a[16*" #B "+11]\n\t"                                \
                   "v_accvgpr_read_b32 %12, a[16*" #B "+12]\n\t"                                \
                   "v_accvgpr_read_b32 %13, a[16*" #B "+13]\n\t"                                \
                   "v_accvgpr_read_b32 %14, a[16*" #B "+14]\n\t"                                \
                   "v_accvgpr_read_b32 %15, a[16*" #B "+15]"                                    \
                   : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]),    \
                     "=v"(x[6]), "=v"(x[7]), "=v"(x[8]), "=v"(x[9]), "=v"(x[10]), "=v"(x[11]),  \
                     "=v"(x[12]), "=v"(x[13]), "=v"(x[14]), "=v"(x[15])                         \
                   :: FA_ACC_CLOBBER_##B);                                                      \
    }                                                                                           \
  };
FA_DEFINE_ACC(0)
FA_DEFINE_ACC(1)
FA_DEFINE_ACC(2)
FA_DEFINE_ACC(3)
FA_DEFINE_ACC(4)
FA_DEFINE_ACC(5)
FA_DEFINE_ACC(6)
FA_DEFINE_ACC(7)
#undef FA_DEFINE_ACC
#undef FA_ACC_RANGE

// Waits for every matrix instruction in flight to have written its
// accumulators (32 wait states cover the longest 32x32 instruction).
__device__ __forceinline__ void acc_drain() { asm volatile("s_nop 15\n\ts_nop 15"); }
// Two wait states after accumulator writes, before a matrix instruction
// reads them as srcC.
__device__ __forceinline__ void acc_settle() { asm volatile("s_nop 2"); }

__device__ __forceinline__ void acc_zero_all() {
  Acc<0>::zero(); Acc<1>::zero(); Acc<2>::zero(); Acc<3>::zero();
  Acc<4>::zero(); Acc<5>::zero(); Acc<6>::zero(); Acc<7>::zero();
}

// O rescale of the lazy reference: row group t by alpha[t].
__device__ __forceinline__ void acc_rescale(const float (&alpha)[NT]) {
  acc_drain();
  Acc<0>::scale(alpha[0]); Acc<1>::scale(alpha[0]); Acc<2>::scale(alpha[0]);
  Acc<3>::scale(alpha[0]);
  Acc<4>::scale(alpha[1]); Acc<5>::scale(alpha[1]); Acc<6>::scale(alpha[1]);
  Acc<7>::scale(alpha[1]);
  acc_settle();
}

// P V products of one 16-key step u of a 32-key sub-tile for head-dim block
// DT: the V^T fragment feeds both row groups.
template <int DT>
__device__ __forceinline__ void pv_pair(bf16x8 v, bf16x8 p0, bf16x8 p1) {
  Acc<DT>::mfma(v, p0);
  Acc<4 + DT>::mfma(v, p1);
}

__device__ __forceinline__ void pv_pair_dt(int dt, bf16x8 v, bf16x8 p0, bf16x8 p1) {
  switch (dt) {  // dt is a compile-time constant at every call site
    case 0: pv_pair<0>(v, p0, p1); break;
    case 1: pv_pair<1>(v, p0, p1); break;
    case 2: pv_pair<2>(v, p0, p1); break;
    default: pv_pair<3>(v, p0, p1); break;
  }
}

// ---------------------------------------------------------------------------
// Per-wave state and one 32-key sub-tile's pieces.
// ---------------------------------------------------------------------------

// dst = src through a move whose output is tied to dst's register.  Used
// where a rare branch recomputes values that the common path leaves in
// place: the branch then writes them into the same registers, and the
// merge after it needs no copies on the common path.
__device__ __forceinline__ void tie_assign(float& dst, float src) {
  asm volatile("v_mov_b32 %0, %1" : "+v"(dst) : "v"(src));
}
__device__ __forceinline__ void tie_assign(uint32_t& dst, uint32_t src) {
  asm volatile("v_mov_b32 %0, %1" : "+v"(dst) : "v"(src));
}

template <int V>
struct Parity {
  static constexpr int value = V;
};

struct State {
  bf16x8 qf[NT][D / 16];  // Q^T, B operand of S^T = K Q^T (row group t, k-step st)
  float mc[NT];           // reference r of each lane's row (base 2, times c)
  float l[NT];            // running sum of this half-wave's probabilities
};

// Sets to -inf every score of a 32-key sub-tile whose key offset (minus 4 hh)
// exceeds lim[t]; offsets are (v & 3) + 8 (v >> 2).
__device__ __forceinline__ void mask_sub(f32x16 (&s)[NT], const int (&lim)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if ((v & 3) + 8 * (v >> 2) > lim[t]) s[t][v] = -INFINITY;
}

// S^T of one 32-key sub-tile (tile rows 32 KT..) for both row groups; every K
// fragment feeds two products.
template <int KT>
__device__ __forceinline__ void scores_sub(f32x16 (&s)[NT], const char* __restrict__ k_st,
                                           const LdsRead<D>& rd, const State& st) {
  bf16x8 a = rd.k(k_st, KT, 0);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 cur = a;
    if (ks + 1 < D / 16) a = rd.k(k_st, KT, ks + 1);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      s[t] = mfma_32x32x16(cur, st.qf[t][ks], ks == 0 ? f32x16{} : s[t]);
  }
}

// O^T += V^T P^T for one 32-key sub-tile, both row groups.
template <int KT>
__device__ __forceinline__ void pv_sub(const char* __restrict__ v_st, const LdsRead<D>& rd,
                                       const bf16x8 (&p)[NT][2]) {
  bf16x8 a = rd.v(v_st, KT, 0, 0);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const bf16x8 cur = a;
    if (n + 1 < 8) a = rd.v(v_st, KT, (n + 1) >> 2, (n + 1) & 3);
    pv_pair_dt(n & 3, cur, p[0][n >> 2], p[1][n >> 2]);
  }
}

// Row-maximum path of the online softmax for one sub-tile: moves a row's
// reference to its new maximum when that exceeds the old one by more than
// kRescaleTau, forms the probabilities against it, and returns whether any
// row of the wave moved (alpha then holds the rescale factors).
__device__ __forceinline__ bool softmax_max_path(State& st, const f32x16 (&s)[NT],
                                                 bf16x8 (&p)[NT][2], float (&alpha)[NT],
                                                 float c) {
  bool moved = false;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[t][v]);
    const float mx_c = halfwave_max(mx) * c;
    const float mref = (mx_c > st.mc[t] + kRescaleTau) ? mx_c : st.mc[t];
    moved |= mref != st.mc[t];
    // a row that has seen only masked keys keeps r = -inf: subtract 0 then
    const float msub = (mref == -INFINITY) ? 0.f : mref;
    alpha[t] = fast_exp2(st.mc[t] - msub);
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float pr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pr[e] = fast_exp2(fmaf(s[t][8 * u + e], c, -msub));
        rs += pr[e];
      }
      p[t][u] = pack_bf16x8(pr);
    }
    st.l[t] = fmaf(alpha[t], st.l[t], rs);
    st.mc[t] = mref;
  }
  return __any(moved);
}

// The row-maximum path writing the packed bf16 pairs of the probabilities
// (pk[t][k] holds elements 2k, 2k+1 of row group t), the registers the
// steady step's accepted path fills, so both paths end in the same place.
__device__ __forceinline__ bool softmax_max_path_pk(State& st, const f32x16 (&s)[NT],
                                                    uint32_t (&pk)[NT][8], float (&alpha)[NT],
                                                    float c) {
  bool moved = false;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[t][v]);
    const float mx_c = halfwave_max(mx) * c;
    const float mref = (mx_c > st.mc[t] + kRescaleTau) ? mx_c : st.mc[t];
    moved |= mref != st.mc[t];
    const float msub = (mref == -INFINITY) ? 0.f : mref;
    alpha[t] = fast_exp2(st.mc[t] - msub);
    float rs = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float p0 = fast_exp2(fmaf(s[t][2 * k], c, -msub));
      const float p1 = fast_exp2(fmaf(s[t][2 * k + 1], c, -msub));
      rs += p0;
      rs += p1;
      pk[t][k] = pack_bf16x2(p0, p1);
    }
    st.l[t] = fmaf(alpha[t], st.l[t], rs);
    st.mc[t] = mref;
  }
  return __any(moved);
}

// Masks S(j+1) at the end of a sub-step, each element moved back into its
// own register (the mask runs on a rare branch; see tie_assign).
__device__ __forceinline__ void mask_sub_tied(f32x16 (&s)[NT], const int (&lim)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float e = s[t][v];
      tie_assign(e, ((v & 3) + 8 * (v >> 2) > lim[t]) ? -INFINITY : e);
      s[t][v] = e;
    }
}

// One steady sub-step j of a wave (1 <= j <= n_w - 2):
//   S(j+1) = K_{j+1} Q^T          16 products, K fragment shared by the groups
//   O     += P(j-1) V_{j-1}       16 products into the AGPR accumulators
//   P(j)   = softmax of S(j)      32 probabilities per lane
// With one wave per SIMD nothing else hides a stall, so the step is laid out
// as 32 slots of one matrix instruction each, alternating score and P V
// products, and every slot issues the ALU work of the probabilities in
// flight: the FMA of probability e+1, the exponential of e, and the row-sum
// add (and bf16 pack) of e-1.  None of a slot's ALU instructions depends on
// another of the same slot, and the slot's product runs while they issue.
//
// The probabilities are formed against the rows' current references with no
// row maximum: p = 2^(s c - r) is at most the lane's sum of them, so when no
// lane's sum exceeds kSumCap (and none is inf or NaN) the references stay.
// Otherwise the scores of S(j), kept unchanged, take the row-maximum path,
// and O (which then holds the P V products up to block j-1) is rescaled at
// once.  S(j) arrives masked; S(j+1) is masked here when it crosses the end
// of the keys or the wave's diagonal (masked_next).  The three rare cases
// share one branch at the end of the step.
//
// kf0 / vf0 carry the first K and V fragments of a sub-step, read by the
// sub-step before, so that their LDS latency hides under its products.  The
// first sub-step of a period (KT = 0) reads those of the second; the second
// (KT = 1) runs `stage` after its last fragment read, which waits for the
// next period's tiles, meets the workgroup at its barrier and starts the
// loads after them, and then reads that period's first fragments.
template <int KT, typename Stage>
__device__ __forceinline__ void steady_sub(State& st, const char* __restrict__ k_st,
                                           const char* __restrict__ v_st, const LdsRead<D>& rd,
                                           const f32x16 (&sc)[NT], f32x16 (&sn)[NT],
                                           const bf16x8 (&pp)[NT][2], bf16x8 (&pc)[NT][2],
                                           float c, bool masked_next, const int (&lim_next)[NT],
                                           bf16x8& kf0, bf16x8& vf0, Stage&& stage,
                                           bool do_stage) {
  constexpr int NE = 32;  // probabilities per lane: e = 16 t + v
  float rs[NT] = {0.f, 0.f};
  // packed bf16 pairs, element k & 3 of pw[t][k >> 2] holding elements
  // 2k, 2k+1 of row group t: already the P^T operand tuples of the next step
  u32x4 pw[NT][2];
  float x[NE], pe[NE];
  // fragments: K for score k-step m (slots 4m, 4m+2), V for P V step m (slots
  // 4m+1, 4m+3), each read one k-step ahead.  A slot issues its matrix
  // instruction, then its operand reads, then the softmax work: reads issued
  // behind the ALU instructions of a slot cost the wave several cycles each
  // more than reads issued right after the matrix instruction.
  bf16x8 kf[2], vf[2];
  kf[0] = kf0;
  vf[0] = vf0;
  x[0] = fmaf(sc[0][0], c, -st.mc[0]);
  auto slot = [&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    constexpr int m = i >> 2;
    if constexpr ((i & 3) == 0) {
      sn[0] = mfma_32x32x16(kf[m & 1], st.qf[0][m], m == 0 ? f32x16{} : sn[0]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (m + 1 < 8) kf[(m + 1) & 1] = rd.k(k_st, KT, m + 1);
      if constexpr (m == 7 && KT == 0) kf0 = rd.k(k_st, 1, 0);
    } else if constexpr ((i & 3) == 1) {
      Acc<m & 3>::mfma(vf[m & 1], pp[0][m >> 2]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (m + 1 < 8) vf[(m + 1) & 1] = rd.v(v_st, KT, (m + 1) >> 2, (m + 1) & 3);
      if constexpr (m == 7 && KT == 0) vf0 = rd.v(v_st, 1, 0, 0);
      // slot 29: every operand read of this period's stages has been waited
      // for (the last V fragment before this product, the last K fragment
      // before slot 28's) and none is issued here, so the next period's
      // loads may overwrite them
      if constexpr (i == 29 && KT == 1) {
        if (do_stage) stage(kf0, vf0);
      }
    } else if constexpr ((i & 3) == 2) {
      sn[1] = mfma_32x32x16(kf[m & 1], st.qf[1][m], m == 0 ? f32x16{} : sn[1]);
    } else {
      Acc<4 + (m & 3)>::mfma(vf[m & 1], pp[1][m >> 2]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (i + 1 < NE)
      x[i + 1] = fmaf(sc[(i + 1) >> 4][(i + 1) & 15], c, -st.mc[(i + 1) >> 4]);
    pe[i] = fast_exp2(x[i]);
    if constexpr (i >= 1) {
      constexpr int e = i - 1;
      rs[e >> 4] += pe[e];
      if constexpr (e & 1) {
        constexpr int k = (e & 15) >> 1;
        pw[e >> 4][k >> 2][k & 3] = pack_bf16x2(pe[e - 1], pe[e]);
        asm volatile("" ::"v"(pw[e >> 4][k >> 2][k & 3]));  // keep the pack in its slot
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(rs[t]));
    __builtin_amdgcn_sched_barrier(0);
  };
  static_for<NE>(slot);
  rs[1] += pe[NE - 1];
  pw[1][1][3] = pack_bf16x2(pe[NE - 2], pe[NE - 1]);

  const bool ok = rs[0] <= kSumCap && rs[1] <= kSumCap;
  const bool all_ok = __all(ok);
  if (__builtin_expect(all_ok && !masked_next, 1)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) tie_assign(st.l[t], st.l[t] + rs[t]);
  } else {
    if (all_ok) {
#pragma unroll
      for (int t = 0; t < NT; ++t) tie_assign(st.l[t], st.l[t] + rs[t]);
    } else {
      // the row-maximum path, its results moved into the registers the
      // accepted path fills; O is rescaled now, before P(j) V_j
      State s2 = st;
      uint32_t pk2[NT][8];
      float alpha[NT];
      const bool moved = softmax_max_path_pk(s2, sc, pk2, alpha, c);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        tie_assign(st.l[t], s2.l[t]);
        tie_assign(st.mc[t], s2.mc[t]);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          uint32_t w = pw[t][k >> 2][k & 3];
          tie_assign(w, pk2[t][k]);
          pw[t][k >> 2][k & 3] = w;
        }
      }
      if (moved) acc_rescale(alpha);
    }
    if (masked_next) mask_sub_tied(sn, lim_next);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u) pc[t][u] = __builtin_bit_cast(bf16x8, pw[t][u]);
}

// A sub-step at the edges of the key loop, phase by phase: j = -1 (clear O,
// S(0)), j = 0 (no P V yet), the last two sub-steps of the wave, and
// sub-steps in which this wave has no key block left while the others of
// its workgroup still do.  Like the steady step it leaves O rescaled to the
// references it ends with, and S(j+1) masked (masked_next).
template <int KT>
__device__ __forceinline__ void general_sub(int j, int n_w, State& st,
                                            const char* __restrict__ k_st,
                                            const char* __restrict__ v_st, const LdsRead<D>& rd,
                                            f32x16 (&sc)[NT], f32x16 (&sn)[NT],
                                            const bf16x8 (&pp)[NT][2], bf16x8 (&pc)[NT][2],
                                            float c, bool masked, const int (&lim)[NT],
                                            bool masked_next, const int (&lim_next)[NT]) {
  if (j < 0) acc_zero_all();
  if (j >= 1 && j - 1 < n_w) {
    // P(j-1) may have been converted just before: two wait states before the
    // matrix instructions read it
    asm volatile("s_nop 1");
    pv_sub<KT>(v_st, rd, pp);
  }
  if (j + 1 < n_w) {
    scores_sub<KT>(sn, k_st, rd, st);
    if (masked_next) mask_sub(sn, lim_next);
  }
  if (j >= 0 && j < n_w) {
    if (masked) mask_sub(sc, lim);
    float alpha[NT];
    if (softmax_max_path(st, sc, pc, alpha, c)) acc_rescale(alpha);
  }
}

// NW waves of 64 rows per workgroup (one wave per SIMD).  A workgroup runs
// the query tiles of blocks t = blockIdx.x, blockIdx.x + gridDim.x, ... in
// turn (the host launches one workgroup per tile, or fewer so that each
// runs several); PAIR gives each block two causal query tiles, n-1-i then
// i.  Before a tile's epilogue the workgroup starts the next tile's Q loads
// and first K stage, so that their latency passes under the epilogue and
// its stores.
template <int NW, bool CAUSAL, bool PAIR>
__device__ __forceinline__ void wide_body(const FwdParams& p) {
  constexpr int BR = NW * 64;
  // K stages 0 and 1, V stages 0 and 1, then one epilogue area per wave
  // (80 KB in all for two waves, so that two such workgroups share a CU)
  __shared__ __attribute__((aligned(1024))) char lds[4 * STG_BYTES + NW * kEpiBytes];
  const uint32_t lds_base = lds_address(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m32 = lane & 31, hh = lane >> 5;
  const size_t q_stride = (size_t)p.hq * D;
  const size_t kv_stride = (size_t)p.hkv * D;

  TileDMA<D, STG, NW> dma;
  dma.init(kv_stride, wave, lane);
  // LDS address of this wave's 1 KB in every stage buffer
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds_base + (uint32_t)wave * 1024u);
  LdsRead<D> rd;
  rd.init(lane);

  // One query tile of one (sequence, query head).
  struct Tile {
    int h, q_start, Lq, Lk, qt;
    const uint16_t* kbase;
    const uint16_t* vbase;
  };
  // Task k of the workgroup: block t = blockIdx.x + (k / TPB) gridDim.x, a
  // work item (sequence b, kv head, query head in group, query tile i), and
  // for PAIR its tile n-1-i (k even) or i (k odd).  False when the task has
  // no rows (past a shorter sequence, or the two tiles of a pair coincide).
  constexpr int TPB = PAIR ? 2 : 1;
  auto task = [&](const int k, Tile& T) __attribute__((always_inline)) -> bool {
    const int t = blockIdx.x + (k / TPB) * gridDim.x;
    // xcd_remap with the launch's divisors precomputed (FastDiv)
    int item = t;
    if (t < p.remap_end) {
      const uint32_t slot = (uint32_t)t >> 3;
      const uint32_t r = p.fd_gs.div(slot);
      item = (int)((r * 8 + ((uint32_t)t & 7)) * p.fd_gs.d + (slot - r * p.fd_gs.d));
    }
    uint32_t rest = p.fd_items.div((uint32_t)item);
    const int it = item - (int)(rest * p.fd_items.d);
    uint32_t next = p.fd_group.div(rest);
    const int hg = (int)(rest - next * p.fd_group.d);
    rest = next;
    next = p.fd_hkv.div(rest);
    const int kvh = (int)(rest - next * p.fd_hkv.d);
    const int b = (int)next;
    T.h = kvh * p.group + hg;
    int k_start;
    if (p.cu_q) {
      T.q_start = p.cu_q[b];
      T.Lq = p.cu_q[b + 1] - T.q_start;
      k_start = p.cu_k[b];
      T.Lk = p.cu_k[b + 1] - k_start;
    } else {
      T.q_start = b * p.seqlen_q;
      T.Lq = p.seqlen_q;
      k_start = b * p.seqlen_k;
      T.Lk = p.seqlen_k;
    }
    T.kbase = p.k + (size_t)k_start * kv_stride + (size_t)kvh * D;
    T.vbase = p.v + (size_t)k_start * kv_stride + (size_t)kvh * D;
    // every field is the same in all lanes; saying so keeps them in scalar
    // registers (the tile loads take their base from there)
    T.h = __builtin_amdgcn_readfirstlane(T.h);
    T.q_start = __builtin_amdgcn_readfirstlane(T.q_start);
    T.Lq = __builtin_amdgcn_readfirstlane(T.Lq);
    T.Lk = __builtin_amdgcn_readfirstlane(T.Lk);
    T.kbase = uniform_ptr(T.kbase);
    T.vbase = uniform_ptr(T.vbase);
    if constexpr (PAIR) {
      // tile n-1-i (heaviest) then tile i, n counted per sequence, so every
      // block of a sequence gets about the same work
      const int first = (T.Lq + BR - 1) / BR - 1 - it;
      if (first < it) return false;
      if (k % 2 == 0) {
        T.qt = first;
        return true;
      }
      T.qt = it;
      return it < first;
    } else {
      T.qt = it;
      return it * BR < T.Lq;
    }
  };
  // The first task from k on that has rows, or -1 (uniform across the
  // workgroup: every value involved is).
  auto next_task = [&](int k, Tile& T) __attribute__((always_inline)) -> int {
#pragma clang loop unroll(disable)
    for (;; ++k) {
      if (blockIdx.x + (k / TPB) * gridDim.x >= p.total) return -1;
      if (task(k, T)) return k;
    }
  };
  // 32-key sub-tiles of a tile's workgroup (causal: up to its last row's
  // diagonal), and the 64-key stages that hold them
  auto tile_subs = [&](const Tile& T) __attribute__((always_inline)) {
    int n_sub = (T.Lk + SUB - 1) / SUB;
    if (CAUSAL) {
      const int last_key = min(T.Lk - 1, T.qt * BR + BR - 1 + (T.Lk - T.Lq));
      n_sub = last_key < 0 ? 0 : min(n_sub, last_key / SUB + 1);
    }
    return n_sub;
  };

  // A tile's first loads: K stage 0 into buffer 0, and the wave's Q rows
  // (rows past the end repeat the last row: their results are never stored,
  // and nothing waits here for the loads to land).
  auto prefetch = [&](const Tile& T, State& st) __attribute__((always_inline)) {
    if (tile_subs(T) > 0) dma.issue_asm(T.kbase, kv_stride, 0, T.Lk - 1, lds, lds_base, wave, lane);
    const int qw0 = T.qt * BR + wave * 64;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int qi = qw0 + t * 32 + m32;
      const uint16_t* qp =
          p.q + (size_t)(T.q_start + min(qi, T.Lq - 1)) * q_stride + (size_t)T.h * D + 8 * hh;
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        st.qf[t][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * s));
    }
  };

  // The key loop of a tile whose prefetch has been issued.
  auto body = [&](const Tile& T, State& st) __attribute__((always_inline)) {
    const int q0 = T.qt * BR;
    const int delta = T.Lk - T.Lq;  // bottom-right causal offset
    const int n_sub = tile_subs(T);
    const int n_stage = (n_sub + 1) / 2;
    const int qw0 = q0 + wave * 64;
    const bool wave_active = qw0 < T.Lq;
    const int wave_last_key = CAUSAL ? min(T.Lk - 1, qw0 + 63 + delta) : T.Lk - 1;
    // sub-tiles this wave needs (causal: up to its own diagonal)
    const int n_w =
        (wave_active && wave_last_key >= 0) ? min(n_sub, wave_last_key / SUB + 1) : 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      st.mc[t] = -INFINITY;
      st.l[t] = 0.f;
    }
    // Last admissible key of each of the lane's rows minus 4 hh (the lane's key
    // offset inside a sub-tile); sub-tile j masks against row_lim - 32 j.
    int row_lim[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int qi = qw0 + t * 32 + m32;
      row_lim[t] = (CAUSAL ? min(T.Lk - 1, qi + delta) : T.Lk - 1) - 4 * hh;
    }
    // sub-tile j needs a mask when it crosses the end of the keys or (causal)
    // the diagonal of this wave's first row
    auto edge = [&](int j) {
      const int k0 = j * SUB;
      return (k0 + SUB > T.Lk) || (CAUSAL && k0 + SUB - 1 > qw0 + delta);
    };

    // S(j) lives in sA (j even) or sB (j odd), P(j) in pA / pB likewise.
    f32x16 sA[NT], sB[NT];
    bf16x8 pA[NT][2], pB[NT][2];

    // Period J: K stage J (buffer J & 1) and V stage J-1 (buffer (J-1) & 1)
    // are in LDS; sub-steps 2J-1 and 2J form S(2J) and S(2J+1) from the K
    // stage and the P V of blocks 2J-2 and 2J-1 from the V stage, while K
    // stage J+1 and V stage J stream in.
    auto k_stage = [&](int J) __attribute__((always_inline)) { return lds + (J & 1) * STG_BYTES; };
    auto v_stage = [&](int J) __attribute__((always_inline)) {  // V stage J-1 of period J
      return lds + (2 + ((J & 1) ^ 1)) * STG_BYTES;
    };
    auto stage_period = [&](const int J) __attribute__((always_inline)) {
      wait_dma();       // this wave's share of K stage J and V stage J-1 has landed
      __syncthreads();  // everyone's has; K stage J-1 and V stage J-2 are read
      const int par = J & 1;
      if (J + 1 < n_stage)
        dma.issue_asm(T.kbase, kv_stride, (J + 1) * STG, T.Lk - 1, lds + (par ^ 1) * STG_BYTES,
                      lds_base + (par ^ 1) * STG_BYTES, wave, lane);
      if (J < n_stage)
        dma.issue_asm(T.vbase, kv_stride, J * STG, T.Lk - 1, lds + (2 + par) * STG_BYTES,
                      lds_base + (2 + par) * STG_BYTES, wave, lane);
    };
    auto limits = [&](const int j, int (&lim)[NT]) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) lim[t] = row_lim[t] - j * SUB;
    };
    // Edge periods, phase by phase, with the stage parity known at run time.
    auto general_period = [&](const int J) __attribute__((always_inline)) {
      stage_period(J);
      const char* k_st = k_stage(J);
      const char* v_st = v_stage(J);
      int lim0[NT], lim1[NT], lim2[NT];
      limits(2 * J - 1, lim0);
      limits(2 * J, lim1);
      limits(2 * J + 1, lim2);
      general_sub<0>(2 * J - 1, n_w, st, k_st, v_st, rd, sB, sA, pA, pB, p.c, edge(2 * J - 1),
                     lim0, edge(2 * J), lim1);
      general_sub<1>(2 * J, n_w, st, k_st, v_st, rd, sA, sB, pB, pA, p.c, edge(2 * J), lim1,
                     edge(2 * J + 1), lim2);
    };
    // Steady periods (both sub-steps steady for this wave), parity static so
    // that every LDS offset is an instruction immediate.  The first one of a
    // run meets the workgroup at its own start (stage_period).  Each one
    // meets the workgroup for the next from inside its second sub-step and
    // there issues the loads of the period after that (K stage J+2, V stage
    // J+1), a full period ahead of their use.  Those stages either lie wholly
    // inside the keys or wholly past them (last_steady below keeps a stage
    // that straddles the last key out of the steady periods), so the loads
    // take the whole-tile offsets with a scalar base clamped to the last 64
    // rows: a stage past the end rereads those rows into a buffer nobody
    // reads.  No vector arithmetic and no branch per load.
    bf16x8 kf0, vf0;
    constexpr int PW = decltype(dma)::PER_WAVE;
    const int last_whole = T.Lk - STG;  // first row of the last 64 keys
    // instruction n of K stage KS (n < PW) or V stage KS - 1 (n >= PW), into
    // K buffer KB and V buffer 2 + VB
    auto load_part = [&](const int KS, auto nc, auto kbuf, auto vbuf)
        __attribute__((always_inline)) {
      constexpr int n = decltype(nc)::value;
      if constexpr (n < PW) {
        constexpr uint32_t KB = decltype(kbuf)::value;
        const uint16_t* src = T.kbase + (size_t)min(KS * STG, last_whole) * kv_stride;
        dma16_si<KB * STG_BYTES + (uint32_t)(n * NW) * 1024u>(dma.obytes[n], src, lds_wave);
      } else {
        constexpr uint32_t VB = decltype(vbuf)::value;
        const uint16_t* src = T.vbase + (size_t)min((KS - 1) * STG, last_whole) * kv_stride;
        dma16_si<(2 + VB) * STG_BYTES + (uint32_t)((n - PW) * NW) * 1024u>(dma.obytes[n - PW],
                                                                             src, lds_wave);
      }
    };
    auto steady_period = [&](const int J, auto par, const bool staged, const bool stage_next)
        __attribute__((always_inline)) {
      constexpr int PAR = decltype(par)::value;
      const char* k_st = lds + PAR * STG_BYTES;
      const char* v_st = lds + (2 + (PAR ^ 1)) * STG_BYTES;
      if (!staged) {
        stage_period(J);
        kf0 = rd.k(k_st, 0, 0);
        vf0 = rd.v(v_st, 0, 0, 0);
      }
      int lim1[NT], lim2[NT];
      limits(2 * J, lim1);
      limits(2 * J + 1, lim2);
      auto no_stage = [](bf16x8&, bf16x8&) {};
      // the next period's tiles have landed and every wave is done with this
      // period's stages: K stage J+1 and V stage J are in buffers PAR ^ 1 and
      // 2 + PAR; K stage J+2 and V stage J+1 go to buffers PAR and 2 + (PAR ^ 1)
      auto next_stage = [&](bf16x8& kn, bf16x8& vn) __attribute__((always_inline)) {
        wait_dma();
        __syncthreads();
        auto one = [&](auto nc) __attribute__((always_inline)) {
          load_part(J + 2, nc, Parity<PAR>{}, Parity<PAR ^ 1>{});
        };
        static_for<2 * PW>(one);
        kn = rd.k(lds + (PAR ^ 1) * STG_BYTES, 0, 0);
        vn = rd.v(lds + (2 + PAR) * STG_BYTES, 0, 0, 0);
      };
      steady_sub<0>(st, k_st, v_st, rd, sB, sA, pA, pB, p.c, edge(2 * J), lim1, kf0, vf0,
                    no_stage, false);
      steady_sub<1>(st, k_st, v_st, rd, sA, sB, pB, pA, p.c, edge(2 * J + 1), lim2, kf0, vf0,
                    next_stage, stage_next);
    };
    // Sub-steps -1 .. n_sub run in periods 0 .. n_stage.  A sub-step j is
    // steady when 1 <= j <= n_w - 2, so periods 1 .. (n_w - 2) / 2 are.  The
    // steady periods' loads reach K stage last_steady + 1; when the keys end
    // inside stage n_stage - 1, that stage must be loaded by a general
    // period, so the steady ones stop at n_stage - 3.
    const int n_period = n_stage + 1;
    int last_steady = n_w >= 4 ? (n_w - 2) / 2 : 0;
    if (T.Lk % STG != 0) last_steady = max(0, min(last_steady, n_stage - 3));
    general_period(0);
    // the Q loads are known complete from here on (the first steady period
    // waits for this period's tile loads anyway)
    vm_drain();
    int J = 1;
    bool staged = false;
#pragma clang loop unroll(disable)
    while (J + 1 <= last_steady) {
      steady_period(J, Parity<1>{}, staged, true);
      steady_period(J + 1, Parity<0>{}, true, J + 2 <= last_steady);
      staged = true;
      J += 2;
    }
    if (J <= last_steady) {
      steady_period(J, Parity<1>{}, staged, false);
      ++J;
    }
#pragma clang loop unroll(disable)
    for (; J < n_period; ++J) general_period(J);

  };

  // O / l and LSE = ln 2 * (r + log2 l).  The output goes out in pieces of
  // 32 rows x 256 bytes (a row group's whole bf16 rows, or half of its fp32
  // rows) through this wave's 8 KB epilogue area, so that every global store
  // writes 16-byte chunks of one contiguous 256-byte run: row r of a piece
  // holds its 16 chunks XOR-swizzled by r & 15, which keeps both the writes
  // and the row reads free of bank conflicts.  Only this wave uses its area.
  auto epilogue = [&](const Tile& T, const State& st) __attribute__((always_inline)) {
    const int qw0 = T.qt * BR + wave * 64;
    char* stg = lds + 4 * STG_BYTES + wave * kEpiBytes;
    const bool f32 = p.o_f32 != 0;
    const size_t esz = f32 ? 4 : 2;                // bytes per output value
    const size_t o_row = (size_t)p.hq * D * esz;  // bytes per token
    const int c = lane & 15;
    // The lane stores row 4 i + (lane >> 4) of a piece at o_lane + (32 t +
    // 4 i) o_row + 256 piece: one per-lane product per tile, and a constant
    // multiple of the uniform row pitch per store.
    char* const o_lane = reinterpret_cast<char*>(p.o) +
                         (size_t)(T.q_start + qw0 + (lane >> 4)) * o_row +
                         (size_t)T.h * D * esz + 16 * c;
    // Rows that exist from the lane's first row on.  Every row of a wave whose
    // 64 rows are all inside the sequence exists, and its stores test nothing.
    const int rows_left = T.Lq - qw0 - (lane >> 4);
    const bool full = qw0 + 64 <= T.Lq;
    // rows back out, 16 bytes per lane, 4 rows per wave instruction.  The
    // stores are non-temporal: O is not read again by this launch, and lines
    // streamed out of L2 as they are written leave less dirty data for the
    // write-back at the end of the kernel (measured: 1 µs less per launch).
    auto store_piece = [&](const int t, const int piece) __attribute__((always_inline)) {
      u32x4 w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4);
        w[i] = *reinterpret_cast<const u32x4*>(stg + r * 256 + ((c ^ (r & 15)) << 4));
      }
      char* const op = o_lane + (size_t)(32 * t) * o_row + 256 * piece;
      if (full) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          __builtin_nontemporal_store(w[i], reinterpret_cast<u32x4*>(op + (size_t)(4 * i) * o_row));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (32 * t + 4 * i < rows_left)
            __builtin_nontemporal_store(w[i],
                                        reinterpret_cast<u32x4*>(op + (size_t)(4 * i) * o_row));
      }
    };
    auto read_block = [&](const int b, float (&x)[16]) __attribute__((always_inline)) {
      switch (b) {
        case 0: Acc<0>::read(x); break;
        case 1: Acc<1>::read(x); break;
        case 2: Acc<2>::read(x); break;
        case 3: Acc<3>::read(x); break;
        case 4: Acc<4>::read(x); break;
        case 5: Acc<5>::read(x); break;
        case 6: Acc<6>::read(x); break;
        default: Acc<7>::read(x); break;
      }
    };
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float lt = halfwave_sum(st.l[t]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse = lt > 0.f ? (st.mc[t] + __log2f(lt)) * kLn2 : -INFINITY;
      const int qi = qw0 + t * 32 + m32;
      if (qi < T.Lq && hh == 0) p.lse[(size_t)(T.q_start + qi) * p.hq + T.h] = lse;
      // the lane holds head-dim dt*32 + 8g + 4hh + 0..3 of row m32 in block
      // 4t + dt, values 4g .. 4g+3
      if (f32) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          float x[16];
          read_block(4 * t + dt, x);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            // fp32 pieces hold head-dim blocks dt = 2 piece, 2 piece + 1
            const int ch = (dt & 1) * 8 + 2 * g + hh;
            const f32x4 w = {x[4 * g] * inv, x[4 * g + 1] * inv, x[4 * g + 2] * inv,
                             x[4 * g + 3] * inv};
            *reinterpret_cast<f32x4*>(stg + m32 * 256 + ((ch ^ (m32 & 15)) << 4)) = w;
          }
          if (dt & 1) store_piece(t, dt >> 1);
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          float x[16];
          read_block(4 * t + dt, x);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int ch = dt * 4 + g;  // 16-byte chunk of the 256-byte row, half hh
            const u32x2 w = {pack_bf16x2(x[4 * g] * inv, x[4 * g + 1] * inv),
                             pack_bf16x2(x[4 * g + 2] * inv, x[4 * g + 3] * inv)};
            *reinterpret_cast<u32x2*>(stg + m32 * 256 + ((ch ^ (m32 & 15)) << 4) + 8 * hh) = w;
          }
        }
        store_piece(t, 0);
      }
    }
  };

  Tile cur;
  int k = next_task(0, cur);
  if (k < 0) return;
  State st;
  prefetch(cur, st);
#pragma clang loop unroll(disable)
  while (true) {
    body(cur, st);
    Tile nxt;
    const int kn = next_task(k + 1, nxt);
    acc_drain();
    __syncthreads();  // every wave is done reading the K/V stages
    // the next tile's Q goes to st.qf, which the epilogue does not read
    if (kn >= 0) prefetch(nxt, st);
    epilogue(cur, st);
    if (kn < 0) break;
    cur = nxt;
    k = kn;
  }
}

}  // namespace wide

template <int NW, bool CAUSAL, bool PAIR>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1)))
void fwd_wide_kernel(const FwdParams p) {
  wide::wide_body<NW, CAUSAL, PAIR>(p);
}

template __global__ void fwd_wide_kernel<4, false, false>(const FwdParams);
template __global__ void fwd_wide_kernel<2, false, false>(const FwdParams);
template __global__ void fwd_wide_kernel<4, true, true>(const FwdParams);
template __global__ void fwd_wide_kernel<2, true, true>(const FwdParams);

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

// Compute units of the current device (0 if unknown), looked up once.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return 0;
    g_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

hipError_t launch_fwd_wide(const FwdParams& p, bool causal, hipStream_t stream) {
  // Each wave takes a whole SIMD, so 4 / waves workgroups fill a compute
  // unit.  A fixed-length batch, whose blocks all cost the same (one tile,
  // or a causal pair of a heavy and a light tile), launches just enough
  // workgroups to fill every compute unit once, each taking every (grid)-th
  // block, so that a tile's first loads overlap the previous tile's
  // epilogue.  A multiple of 8 workgroups keeps every tile of a
  // workgroup on the same XCD as its block index.  Packed sequences keep one
  // workgroup per tile, which the hardware hands out as compute units free up.
  int grid = p.total;
  const int slots = (device_cus() & ~7) * (4 / p.waves);
  if (!p.cu_q && slots > 0 && grid > slots) grid = slots;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(p.waves * 64), 0, stream, p);
    return hipGetLastError();
  };
  if (causal)
    return p.waves == 4 ? go(fwd_wide_kernel<4, true, true>) : go(fwd_wide_kernel<2, true, true>);
  return p.waves == 4 ? go(fwd_wide_kernel<4, false, false>)
                      : go(fwd_wide_kernel<2, false, false>);
}

}  // namespace fa
