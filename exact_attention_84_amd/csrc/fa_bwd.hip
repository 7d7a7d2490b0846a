// Backward of the fused attention: the gradients dQ, dK, dV of <dO, O>.
//
// The forward keeps only O and the per-row logsumexp; the backward recomputes
// P = exp2(S c - LSE log2(e)) tile by tile instead of storing it, and splits
// the work by key blocks so that dK and dV accumulate on chip
// ("FlashAttention — IO 感知的精确注意力 kernel", section 4: recompute P from
// the saved logsumexp, change the parallel axis for the backward; section 2.2:
// the backward kernel recomputes P and accumulates dK/dV).  With
// D = rowsum(dO * O) (the same page's preprocess step, section 7):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,
//   dK = scale dS^T Q.
// Three kernels:
//   preprocess  D and LSE * log2(e) per query row and head, head-major;
//   dK/dV       one workgroup per (sequence, kv head, block of keys): this
//               lane's key row of K and V stays in registers, Q and dO tiles
//               of every query head of the group stream through LDS, and the
//               group's gradients are summed on chip (no atomics);
//   dQ          one workgroup per (sequence, query head, tile of query rows):
//               Q and dO stay in registers, K and V tiles stream through LDS.
// The page's kernel adds dQ with atomics, which makes the backward
// nondeterministic (its section 5); computing dQ in its own pass keeps this
// one bitwise reproducible.
//
// Every product reuses the forward's two MFMA shapes: scores_tile (A = rows of
// an LDS tile, B = fragments in registers) gives S^T = K Q^T and
// dP^T = V dO^T in the dQ pass, S = Q K^T and dP = dO V^T in the dK/dV pass;
// pv_tile (A = an LDS tile read transposed, B = bf16 probabilities in the
// accumulator order) gives dQ^T += K^T dS^T, dV^T += dO^T P and
// dK^T += Q^T dS.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.hpp"


namespace fa {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// D[h][r] = sum_d dO[r][h][d] O[r][h][d] and LSE[r][h] log2(e), one group of
// D/8 lanes per (row, head).  Workspace rows past the last query row (up to
// the padded stride) get D = 0 and LSE log2(e) = +inf, so a tile that reads
// past its sequence sees P = 0 and finite D there.
template <int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const BwdParams p) {
  constexpr int LPP = D / 8;
  constexpr int PPB = 256 / LPP;
  const int tid = threadIdx.x;
  const long long pair = (long long)blockIdx.x * PPB + tid / LPP;
  const int sub = tid % LPP;
  const int h = (int)(pair % p.hq);
  const long long r = pair / p.hq;
  long long rows = p.cu_q ? p.cu_q[p.batch] : (long long)p.batch * p.seqlen_q;
  rows = rows < p.rows_cap ? rows : p.rows_cap;
  const bool valid = r < rows;
  float acc = 0.f;
  if (valid) {
    const size_t off = ((size_t)r * p.hq + h) * D + sub * 8;
    const u32x4 a = *reinterpret_cast<const u32x4*>(p.dout + off);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p.o + off);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = fmaf(bf16_lo(a[i]), bf16_lo(b[i]), fmaf(bf16_hi(a[i]), bf16_hi(b[i]), acc));
  }
#pragma unroll
  for (int m = LPP / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (sub == 0 && r < p.ws_stride) {
    const size_t w = (size_t)h * p.ws_stride + r;
    p.dsum[w] = acc;  // 0 past the rows
    p.lse2[w] = valid ? p.lse[(size_t)r * p.hq + h] * kLog2e : INFINITY;  // -inf stays -inf
  }
}

// LDS byte address of a pointer into a __shared__ array, held in a VGPR the
// compiler cannot see through: operand addresses are then formed as this
// register plus the lane's offset, with the sub-tile offset folded into the
// instruction's immediate (one add per read instead of two).
typedef __attribute__((address_space(3))) const char lds_cchar;
__device__ __forceinline__ uint32_t lds_base(const char* p) {
  uint32_t a = (uint32_t)(uintptr_t)(lds_cchar*)p;
  asm volatile("" : "+v"(a));
  return a;
}
template <typename T>
__device__ __forceinline__ T lds_load(uint32_t a) {
  return *(const __attribute__((address_space(3))) T*)(uintptr_t)a;
}
typedef short s16x4b __attribute__((ext_vector_type(4)));
typedef short s16x8b __attribute__((ext_vector_type(8)));

// Per-lane operand base addresses of one swizzled tile, each an opaque VGPR,
// so that every read is a single LDS instruction with the sub-tile / row-step
// offset in its immediate.
template <int D>
struct KBases {  // score operand (rows kt*32 + lane%32, head-dim step st)
  uint32_t b[D / 16];
  __device__ __forceinline__ KBases(uint32_t t, const LdsRead<D>& rd) {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      b[st] = t + rd.kb[st];
      asm volatile("" : "+v"(b[st]));
    }
  }
  __device__ __forceinline__ bf16x8 read(int kt, int st) const {
    return lds_load<bf16x8>(b[st] + kt * 64 * D);
  }
};
template <int D>
struct VBases {  // transposed operand (head-dim block dt, 16-row step (kt, u))
  uint32_t b[D / 32][2];
  __device__ __forceinline__ VBases(uint32_t t, const LdsRead<D>& rd) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        b[dt][sec] = t + rd.vb[dt][sec];
        asm volatile("" : "+v"(b[dt][sec]));
      }
  }
  __device__ __forceinline__ bf16x8 read(int kt, int u, int dt) const {
    const uint32_t row = (kt * 32 + 16 * u) * 2 * D;
    const s16x4b lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4b*)(uintptr_t)(b[dt][0] + row));
    const s16x4b hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4b*)(uintptr_t)(b[dt][1] + row));
    const s16x8b w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
  }
};

// The backward's MFMA sequences, with their LDS operands read two MFMAs
// ahead (LDS latency is longer than one 32-cycle MFMA).
//
// scores_pf: X_kt = A_kt B^T for the NKT 32-row sub-tiles of a swizzled LDS
// tile (A) and a fragment in registers (B), the sub-tiles' chains
// interleaved.
template <int D, int NKT>
__device__ __forceinline__ void scores_pf(f32x16 (&x)[NKT][1], const char* __restrict__ lds,
                                          const LdsRead<D>& rd, const bf16x8 (&b)[1][D / 16]) {
  constexpr int N = NKT * (D / 16);
  const KBases<D> kb(lds_base(lds), rd);
  bf16x8 op[3];
  auto read = [&](int i) { return kb.read(i % NKT, i / NKT); };
  op[0] = read(0);
  op[1] = read(1);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + 2 < N) op[(i + 2) % 3] = read(i + 2);
    const int kt = i % NKT, st = i / NKT;
    x[kt][0] = mfma_32x32x16(op[i % 3], b[0][st], st == 0 ? f32x16{} : x[kt][0]);
  }
}

// pv_pf: acc^T += A_kt^T P_kt over NKT 32-row sub-tiles of a swizzled LDS
// tile read transposed (A) and bf16 operands in accumulator order (P).
template <int D, int NKT>
__device__ __forceinline__ void pv_pf(f32x16 (&acc)[D / 32], const char* __restrict__ lds,
                                      const LdsRead<D>& rd, const bf16x8 (&pb)[NKT][1][2]) {
  constexpr int DT = D / 32;
  constexpr int N = NKT * 2 * DT;
  const VBases<D> vb(lds_base(lds), rd);
  bf16x8 op[3];
  auto read = [&](int i) { return vb.read(i / (2 * DT), (i / DT) & 1, i % DT); };
  op[0] = read(0);
  op[1] = read(1);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + 2 < N) op[(i + 2) % 3] = read(i + 2);
    const int kt = i / (2 * DT), u = (i / DT) & 1, dt = i % DT;
    acc[dt] = mfma_32x32x16(op[i % 3], pb[kt][0][u], acc[dt]);
  }
}

// pv_pf with the tile's transposed-read bases computed once by the caller;
// `off` (a compile-time constant where it is called) selects the stage and
// lands in the instructions' immediates.
template <int D, int NKT>
__device__ __forceinline__ void pv_pf_at(f32x16 (&acc)[D / 32], const VBases<D>& vb, uint32_t off,
                                         const bf16x8 (&pb)[NKT][1][2]) {
  constexpr int DT = D / 32;
  constexpr int N = NKT * 2 * DT;
  bf16x8 op[3];
  auto read = [&](int i) {
    const int kt = i / (2 * DT), u = (i / DT) & 1, dt = i % DT;
    const uint32_t row = off + (kt * 32 + 16 * u) * 2 * D;
    const s16x4b lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4b*)(uintptr_t)(vb.b[dt][0] + row));
    const s16x4b hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4b*)(uintptr_t)(vb.b[dt][1] + row));
    const s16x8b w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
  };
  op[0] = read(0);
  op[1] = read(1);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + 2 < N) op[(i + 2) % 3] = read(i + 2);
    const int kt = i / (2 * DT), u = (i / DT) & 1, dt = i % DT;
    acc[dt] = mfma_32x32x16(op[i % 3], pb[kt][0][u], acc[dt]);
  }
}

// Two independent 32 x 32 score products over the head dimension, their
// MFMA chains interleaved: x = A_x B_x^T and y = A_y B_y^T with A_x, A_y rows
// of swizzled LDS tiles and B_x, B_y fragments in registers.  Operands are
// read two MFMAs ahead.
template <int D>
__device__ __forceinline__ void scores_pair(f32x16& x, f32x16& y, const char* __restrict__ ax,
                                            const char* __restrict__ ay, const LdsRead<D>& rd,
                                            const bf16x8 (&bx)[D / 16],
                                            const bf16x8 (&by)[D / 16]) {
  constexpr int N = 2 * (D / 16);  // MFMAs, alternating x and y
  const KBases<D> kx(lds_base(ax), rd), ky(lds_base(ay), rd);
  bf16x8 op[3];
  auto read = [&](int i) { return (i & 1) ? ky.read(0, i >> 1) : kx.read(0, i >> 1); };
  op[0] = read(0);
  op[1] = read(1);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + 2 < N) op[(i + 2) % 3] = read(i + 2);
    const int st = i >> 1;
    if (i & 1) y = mfma_32x32x16(op[i % 3], by[st], st == 0 ? f32x16{} : y);
    else x = mfma_32x32x16(op[i % 3], bx[st], st == 0 ? f32x16{} : x);
  }
}

// scores_pair with both tiles read through one set of bases computed once
// by the caller, at offsets ox and oy (compile-time constants where it is
// called, so they land in the instructions' immediates).
template <int D>
__device__ __forceinline__ void scores_pair_at(f32x16& x, f32x16& y, const KBases<D>& kb,
                                               uint32_t ox, uint32_t oy,
                                               const bf16x8 (&bx)[D / 16],
                                               const bf16x8 (&by)[D / 16]) {
  constexpr int N = 2 * (D / 16);  // MFMAs, alternating x and y
  bf16x8 op[3];
  auto read = [&](int i) {
    return lds_load<bf16x8>(kb.b[i >> 1] + ((i & 1) ? oy : ox));
  };
  op[0] = read(0);
  op[1] = read(1);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + 2 < N) op[(i + 2) % 3] = read(i + 2);
    const int st = i >> 1;
    if (i & 1) y = mfma_32x32x16(op[i % 3], by[st], st == 0 ? f32x16{} : y);
    else x = mfma_32x32x16(op[i % 3], bx[st], st == 0 ? f32x16{} : x);
  }
}

// dS^T = P^T * (dP^T - D) for NKT 32-key sub-tiles of one wave's rows (lanes),
// rounded to bf16 in the order of the dQ product's B operand.  `lim` is the
// last admissible key of the lane's row relative to the first sub-tile, minus
// the lane's key offset; rows without data are zeroed.
template <int NKT>
__device__ __forceinline__ void dq_scores(const f32x16 (&s)[NKT][1], const f32x16 (&dp)[NKT][1],
                                          bf16x8 (&dsb)[NKT][1][2], int lim, bool row_ok,
                                          float lse2, float dsum, float c, bool masked = true) {
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    float ds[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float pe = fast_exp2(fmaf(s[kt][0][v], c, -lse2));
      const float d = pe * (dp[kt][0][v] - dsum);
      // masked is false only when every row and key of the sub-tiles is
      // admissible (uniform across the wave), and the selects drop out
      ds[v] = (!masked || (row_ok && 32 * kt + (v & 3) + 8 * (v >> 2) <= lim)) ? d : 0.f;
    }
    dsb[kt][0][0] = pack_bf16x8(ds);
    dsb[kt][0][1] = pack_bf16x8(ds + 8);
  }
}

// ---------------------------------------------------------------------------
// dQ: the forward's decomposition.  Each wave owns 32 query rows (one per lane
// column of the accumulators); per 32-key sub-tile it forms S^T = K Q^T and
// dP^T = V dO^T, then dS^T = P^T * (dP^T - D) in registers and
// dQ^T += K^T dS^T.
// ---------------------------------------------------------------------------
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(const BwdParams p) {
  constexpr int BC = 64;
  constexpr int BR = NW * 32;
  constexpr int TILE = BC * D * 2;
  constexpr int KS = D / 16;
  // K stages 0 and 1, then V stages 0 and 1, in one array so that a stage is
  // a constant offset from one set of per-lane read bases
  __shared__ __attribute__((aligned(1024))) char kv_lds[4 * TILE];
  char* const k_lds0 = kv_lds;
  char* const k_lds1 = kv_lds + TILE;
  char* const v_lds0 = kv_lds + 2 * TILE;
  char* const v_lds1 = kv_lds + 3 * TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m32 = lane & 31, hh = lane >> 5;

  // Work item: (sequence b, kv head, query head in group) and query tile qt.
  // Causal tiles cost in proportion to qt + 1, so blocks take them heaviest
  // first over all heads (block w: tile rank w / heads, head w % heads); the
  // hardware hands blocks out in order as compute units free up, and the
  // light tiles fill the gaps the heavy ones leave.  Either way the heads of
  // one kv group, which read the same K and V, share an XCD.
  const int nh = p.batch * p.hq;
  int it, rest;
  if (CAUSAL) {
    const int u = blockIdx.x % nh;
    it = blockIdx.x / nh;
    rest = xcd_remap(u, nh, p.group);
  } else {
    const int item = xcd_remap(blockIdx.x, nh * p.n_qtiles, p.group * p.n_qtiles);
    it = item % p.n_qtiles;
    rest = item / p.n_qtiles;
  }
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
  const int qt = CAUSAL ? p.n_qtiles - 1 - it : it;
  const int q0 = qt * BR;
  if (q0 >= Lq) return;  // packed sequence shorter than this tile (uniform)

  const int delta = Lk - Lq;  // bottom-right causal offset
  int n_kt = (Lk + BC - 1) / BC;
  if (CAUSAL) {
    const int last_key = min(Lk - 1, q0 + BR - 1 + delta);
    n_kt = last_key < 0 ? 0 : min(n_kt, last_key / BC + 1);
  }
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + m32;
  const bool row_ok = qi < Lq && q_start + qi < p.rows_cap;

  const size_t q_stride = (size_t)p.hq * D;
  const size_t kv_stride = (size_t)p.hkv * D;
  WaveState<D, 1> st;  // qf: Q fragments; o: dQ^T accumulator
  st.init();
  bf16x8 dof[1][KS];   // dO fragments
  {
    const size_t off = (size_t)(q_start + qi) * q_stride + (size_t)h * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 rq = {0u, 0u, 0u, 0u}, rd = {0u, 0u, 0u, 0u};
      if (row_ok) {
        rq = *reinterpret_cast<const u32x4*>(p.q + off + 16 * s);
        rd = *reinterpret_cast<const u32x4*>(p.dout + off + 16 * s);
      }
      st.qf[0][s] = __builtin_bit_cast(bf16x8, rq);
      dof[0][s] = __builtin_bit_cast(bf16x8, rd);
    }
  }
  const size_t wrow = (size_t)h * p.ws_stride + q_start + (row_ok ? qi : 0);
  const float lse2 = row_ok ? p.lse2[wrow] : 0.f;
  const float dsum = row_ok ? p.dsum[wrow] : 0.f;
  // last admissible key of this lane's row, minus the lane's key offset 4 hh
  const int row_lim = (CAUSAL ? min(Lk - 1, qi + delta) : Lk - 1) - 4 * hh;

  const uint16_t* kbase = p.k + (size_t)k_start * kv_stride + (size_t)kvh * D;
  const uint16_t* vbase = p.v + (size_t)k_start * kv_stride + (size_t)kvh * D;
  TileDMA<D, BC, NW> dma;
  dma.init(kv_stride, wave, lane);
  LdsRead<D> rd;
  rd.init(lane);
  // K and V tile j into stage s, as asm loads with no branch per instruction
  // (rows clamped to the last key); wait_dma and the barrier order them
  constexpr int PW = decltype(dma)::PER_WAVE;
  const uint32_t kv_row_bytes = 2u * (uint32_t)kv_stride;
  auto load_tiles = [&](const int j, char* k_dst, char* v_dst) {
    const auto ks = decltype(dma)::src(kbase, kv_stride, j * BC, Lk - 1);
    const auto vs = decltype(dma)::src(vbase, kv_stride, j * BC, Lk - 1);
    const uint32_t ka = lds_address(k_dst), va = lds_address(v_dst);
    auto one = [&](auto nc) {
      dma.template issue_one<decltype(nc)::value>(ks, kv_row_bytes, ka, wave);
      dma.template issue_one<decltype(nc)::value>(vs, kv_row_bytes, va, wave);
    };
    static_for<PW>(one);
  };
  if (n_kt > 0) load_tiles(0, k_lds0, v_lds0);
  const int wave_last_key = CAUSAL ? min(Lk - 1, qw0 + 31 + delta) : Lk - 1;
  // Q, dO and the row statistics are known loaded from here on: the
  // compiler then places no waits for them inside the loop, where the
  // counter also counts the asm tile loads
  vm_drain();

  // every row of this wave exists (no row masks); a 32-key sub-tile whose
  // last key every row of the wave admits then needs no mask at all
  const bool rows_all = qw0 + 32 <= min(Lq, p.rows_cap - q_start);
  const int wave_min_key = CAUSAL ? min(Lk - 1, qw0 + delta) : Lk - 1;
  // Step j: K_j, V_j in stage j & 1.  The loop runs steps in pairs so that
  // each step's stage buffers are known at compile time (their offsets are
  // instruction immediates).
  // per-lane read bases of the whole array, computed once: the score reads
  // (K and V tiles alike) and the transposed reads of K
  const KBases<D> kbase_rd(lds_base(kv_lds), rd);
  const VBases<D> vbase_rd(lds_base(kv_lds), rd);
  auto step = [&](const int j, const uint32_t ko, const uint32_t vo, char* kn, char* vn)
      __attribute__((always_inline)) {
    wait_dma();
    __syncthreads();  // K_j, V_j have landed; everyone is done with the other stage
    if (j + 1 < n_kt) load_tiles(j + 1, kn, vn);
    if (qw0 >= Lq) return;  // this wave has no rows (uniform)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int ksub = j * BC + 32 * kt;
      if (ksub > wave_last_key) break;  // past this wave's keys (uniform)
      f32x16 s[1][1], dp[1][1];
      scores_pair_at<D>(s[0][0], dp[0][0], kbase_rd, ko + kt * 64 * D, vo + kt * 64 * D, st.qf[0],
                        dof[0]);
      bf16x8 dsb[1][1][2];
      const bool masked = !rows_all || ksub + 31 > wave_min_key;
      if (masked)
        dq_scores<1>(s, dp, dsb, row_lim - ksub, row_ok, lse2, dsum, p.c, true);
      else
        dq_scores<1>(s, dp, dsb, row_lim - ksub, row_ok, lse2, dsum, p.c, false);
      pv_pf_at<D, 1>(st.o[0], vbase_rd, ko + kt * 64 * D, dsb);  // dQ^T += K^T dS^T
    }
  };
  int j = 0;
#pragma clang loop unroll(disable)
  for (; j + 1 < n_kt; j += 2) {
    step(j, 0, 2 * TILE, k_lds1, v_lds1);
    step(j + 1, TILE, 3 * TILE, k_lds0, v_lds0);
  }
  if (j < n_kt) step(j, 0, 2 * TILE, k_lds1, v_lds1);
  // dQ goes out through this wave's part of the K/V stages (free once every
  // wave is past its last product), as whole 16-byte chunks of row runs
  __syncthreads();
  const size_t esz = p.g_f32 ? 4 : 2;
  char* const stg = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
  store_rows_lds<D>(st.o[0], p.scale,
                    reinterpret_cast<char*>(p.dq) + ((size_t)(q_start + qw0) * p.hq + h) * D * esz,
                    (size_t)p.hq * D * esz, min(Lq, p.rows_cap - q_start) - qw0, p.g_f32 != 0,
                    stg, lane);
}

// ---------------------------------------------------------------------------
// dK, dV: the workgroup owns BK = 128 keys in four 32-key columns, and each
// column has two waves with split roles (the four "S" waves and the four
// "dP" waves share the SIMDs in pairs).  Per 64-query tile of Q and dO, with
// the rows' LSE log2(e) and D staged alongside in LDS:
//   S wave (K row in registers):  S = Q K^T, P = exp2(S c - LSE log2 e) into
//                                 LDS, dV^T += dO^T P
//   dP wave (V row in registers): dP = dO V^T, then (after the exchange)
//                                 dS = P (dP - D), dK^T += Q^T dS
// Each wave holds one D x 32 accumulator, half of what a wave owning both
// gradients needs, which lets two waves share a SIMD and hide each other's
// elementwise work and LDS latency.  Two barriers per tile: the tile has
// landed, and P has been written.  The dP wave applies each tile's dK product
// one tile late, while its partner computes the next tile's exponentials, so
// the SIMD's matrix unit has work during them; Q tiles are therefore
// triple-buffered.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dkdv_kernel(const BwdParams p) {
  constexpr int NW = 8;
  constexpr int BQ = 64;
  constexpr int BK = 128;
  constexpr int TILE = BQ * D * 2;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(1024))) char q_lds[3][TILE];
  __shared__ __attribute__((aligned(1024))) char do_lds[2][TILE];
  // per stage: LSE log2(e) of the tile's 64 rows, then their D (the DMA
  // instruction fills 1 KB; the second half repeats the first)
  __shared__ __attribute__((aligned(1024))) float st_lds[2][256];
  // P of each column's two 32-row sub-tiles, fp32, in accumulator order:
  // [column][sub-tile][register group][lane] of f32x4
  __shared__ __attribute__((aligned(1024))) f32x4 p_lds[4][2][4][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = wave & 3;
  const bool dp_role = wave >= 4;  // uniform per wave
  const int hh = lane >> 5, m32 = lane & 31;

  // Work item: (sequence b, kv head) and key block kblk.  A causal block
  // costs in proportion to the query tiles below its diagonal, most for
  // block 0, so blocks take them heaviest first over all heads (block w: key
  // block w / heads, head w % heads), as the dQ kernel does.
  const int nkv = p.batch * p.hkv;
  int kblk, rest;
  if (CAUSAL) {
    kblk = blockIdx.x / nkv;
    rest = blockIdx.x % nkv;
  } else {
    const int item = xcd_remap(blockIdx.x, nkv * p.n_kblocks, p.n_kblocks);
    kblk = item % p.n_kblocks;
    rest = item / p.n_kblocks;
  }
  const int kvh = rest % p.hkv;
  const int b = rest / p.hkv;

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
  const int k0 = kblk * BK;
  if (k0 >= Lk) return;  // packed sequence shorter than this block (uniform)
  const int delta = Lk - Lq;
  // rows at or past this bound have no workspace entry (a launch sized for
  // fewer rows than the sequences hold); they are masked like padding
  const int lq_eff = min(Lq, p.rows_cap - q_start);
  const int kw0 = k0 + col * 32;
  const int key = kw0 + m32;
  const bool key_ok = key < Lk;

  const size_t q_stride = (size_t)p.hq * D;
  const size_t kv_stride = (size_t)p.hkv * D;
  // the lane's key row of K (S wave) or V (dP wave); zeros past the end
  // (their gradients are accumulated but never stored)
  bf16x8 frag[1][KS];
  {
    const uint16_t* src = dp_role ? p.v : p.k;
    const size_t off = (size_t)(k_start + key) * kv_stride + (size_t)kvh * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 r = {0u, 0u, 0u, 0u};
      if (key_ok) r = *reinterpret_cast<const u32x4*>(src + off + 16 * s);
      frag[0][s] = __builtin_bit_cast(bf16x8, r);
    }
  }
  WaveState<D, 1> acc;  // o: dV^T (S wave) or dK^T (dP wave)
  acc.init();

  // Queries that see key j satisfy i >= j - delta (causal): start at the tile
  // holding the first query that sees this block's first key.
  const int n_qt = (Lq + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? min(n_qt, max(0, k0 - delta) / BQ) : 0;
  const int per_head = n_qt - qt0;
  const int n_steps = p.group * per_head;

  TileDMA<D, BQ, NW> dma;
  dma.init(q_stride, wave, lane);
  LdsRead<D> rd;
  rd.init(lane);
  auto issue = [&](int step) {
    const int stage = step & 1;
    const int hg = step / per_head, q0 = (qt0 + step % per_head) * BQ;
    const int h = p.group * kvh + hg;
    const size_t head = (size_t)h * D;
    const uint16_t* qb = p.q + (size_t)q_start * q_stride + head;
    const uint16_t* db = p.dout + (size_t)q_start * q_stride + head;
    dma.issue(qb, q_stride, q0, Lq - 1, q_lds[step % 3], wave, lane);
    dma.issue(db, q_stride, q0, Lq - 1, do_lds[stage], wave, lane);
    if (wave == 0) {
      // 16 lanes x 16 bytes per statistic; the row base is clamped so the
      // 64-row read stays inside the workspace (its 64 rows of padding)
      const int r0 = min(q_start + q0, p.ws_stride - BQ);
      const float* src = ((lane & 16) ? p.dsum : p.lse2) + (size_t)h * p.ws_stride + r0 +
                         4 * (lane & 15);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)st_lds[stage], 16, 0, 0);
    }
  };
  if (n_steps > 0) issue(0);

  // The step loop, instantiated once per role so that each role's registers
  // are allocated for its own live values.  Both loops meet the same two
  // barriers per tile.
  auto run = [&](auto role) {
    constexpr bool DPR = decltype(role)::value;
    // bf16 B operands of the accumulator's product: the S wave's P (formed
    // and used within a tile) or the dP wave's dS (formed in one tile, used
    // in the next)
    bf16x8 pk[2][1][2];
    bool have_prev = false;
#pragma clang loop unroll(disable)
    for (int step = 0; step < n_steps; ++step) {
      const int stage = step & 1;
      const char* qc = q_lds[step % 3];
      const char* dc = do_lds[stage];
      const float* stl = st_lds[stage];
      wait_dma();
      __syncthreads();  // this tile has landed; everyone is done with the other stages and P
      const int q0 = (qt0 + step % per_head) * BQ;
      // no key in this column, or every key above the diagonal: the column's
      // two waves only keep the barriers
      const bool active = kw0 < Lk && !(CAUSAL && kw0 > q0 + BQ - 1 + delta);
      const int nsub = min(2, (Lq - q0 + 31) / 32);  // sub-tiles holding rows
      f32x16 x[2][1];  // S (S wave) or dP (dP wave) per sub-tile
      // The next tile's loads are issued while this wave's first products
      // run (issuing them right at the barrier queues all eight waves' loads
      // at once).  The dP wave first applies the previous tile's dK product
      // (its Q tile is still resident: three Q stages), then forms dP; the S
      // wave forms S.  Both score products interleave their two sub-tiles'
      // chains (a missing second sub-tile reads clamped rows; its result is
      // not used).
      if constexpr (DPR) {
        if (have_prev) pv_pf<D, 2>(acc.o[0], q_lds[(step + 2) % 3], rd, pk);
        if (step + 1 < n_steps) issue(step + 1);
        if (active) scores_pf<D, 2>(x, dc, rd, frag);
      } else {
        if (active) scores_pf<D, 2>(x, qc, rd, frag);
        if (step + 1 < n_steps) issue(step + 1);
      }
      if constexpr (!DPR) {
        if (active) {
          const bool full = q0 + BQ - 1 < lq_eff && (!CAUSAL || kw0 + 31 <= q0 + delta);
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            if (kt >= nsub) break;
            const int qsub = q0 + 32 * kt;
            const int lo = key - delta - qsub - 4 * hh;  // first admissible row offset (causal)
            const int hi = lq_eff - 1 - qsub - 4 * hh;   // last row offset with data
            float pe[16];
            auto probs = [&](const bool masked) __attribute__((always_inline)) {
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const f32x4 l2 = *reinterpret_cast<const f32x4*>(stl + 32 * kt + 8 * g + 4 * hh);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int r = (e & 3) + 8 * g;  // row offset of element 4 g + e
                  const float v = fast_exp2(fmaf(x[kt][0][4 * g + e], p.c, -l2[e]));
                  pe[4 * g + e] =
                      (!masked || (r <= hi && (!CAUSAL || r >= lo))) ? v : 0.f;
                }
              }
            };
            // two paths on the uniform edge test, so that interior tiles
            // carry no per-element selects (folded into one path, the
            // compiler made every tile pay for them)
            if (full)
              probs(false);
            else
              probs(true);
#pragma unroll
            for (int g = 0; g < 4; ++g)
              p_lds[col][kt][g][lane] =
                  f32x4{pe[4 * g], pe[4 * g + 1], pe[4 * g + 2], pe[4 * g + 3]};
            pk[kt][0][0] = pack_bf16x8(pe);
            pk[kt][0][1] = pack_bf16x8(pe + 8);
          }
        }
      }
      __syncthreads();  // P of this tile is in LDS
      if constexpr (DPR) {
        have_prev = active;
        if (active) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            if (kt >= nsub) break;
            float ds[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 dd =
                  *reinterpret_cast<const f32x4*>(stl + 64 + 32 * kt + 8 * g + 4 * hh);
              const f32x4 pv = p_lds[col][kt][g][lane];
#pragma unroll
              for (int e = 0; e < 4; ++e) ds[4 * g + e] = pv[e] * (x[kt][0][4 * g + e] - dd[e]);
            }
            pk[kt][0][0] = pack_bf16x8(ds);
            pk[kt][0][1] = pack_bf16x8(ds + 8);
          }
          if (nsub < 2) pk[1][0][0] = pk[1][0][1] = bf16x8{};  // no rows
        }
      } else {
        if (active) {
          if (nsub < 2) pk[1][0][0] = pk[1][0][1] = bf16x8{};  // no rows: contributes nothing
          pv_pf<D, 2>(acc.o[0], dc, rd, pk);  // dV^T += dO^T P
        }
      }
    }
    // the last tile's dK product (its Q tile stays resident)
    if constexpr (DPR) {
      if (have_prev) pv_pf<D, 2>(acc.o[0], q_lds[(n_steps - 1) % 3], rd, pk);
    }
  };
  if (dp_role) run(std::true_type{});
  else run(std::false_type{});

  // dV (S waves) and dK (dP waves) go out through LDS that every wave is done
  // with after the barrier, as whole 16-byte chunks of row runs: 8 KB a wave,
  // the S waves' in the P exchange area, the dP waves' in the Q and dO stages
  __syncthreads();
  const size_t esz = p.g_f32 ? 4 : 2;
  char* const stg = !dp_role ? reinterpret_cast<char*>(&p_lds[col][0][0][0])
                    : col < 3 ? &q_lds[0][0] + col * 8192
                              : &do_lds[0][0];
  store_rows_lds<D>(acc.o[0], dp_role ? p.scale : 1.f,
                    reinterpret_cast<char*>(dp_role ? p.dk : p.dv) +
                        ((size_t)(k_start + kw0) * p.hkv + kvh) * D * esz,
                    (size_t)p.hkv * D * esz, Lk - kw0, p.g_f32 != 0, stg, lane);
}

template __global__ void bwd_preprocess_kernel<128>(const BwdParams);
template __global__ void bwd_preprocess_kernel<64>(const BwdParams);
template __global__ void bwd_dq_kernel<128, 4, false>(const BwdParams);
template __global__ void bwd_dq_kernel<128, 4, true>(const BwdParams);
template __global__ void bwd_dq_kernel<64, 4, false>(const BwdParams);
template __global__ void bwd_dq_kernel<64, 4, true>(const BwdParams);
template __global__ void bwd_dkdv_kernel<128, false>(const BwdParams);
template __global__ void bwd_dkdv_kernel<128, true>(const BwdParams);
template __global__ void bwd_dkdv_kernel<64, false>(const BwdParams);
template __global__ void bwd_dkdv_kernel<64, true>(const BwdParams);

constexpr int kBwdWaves = 4;
int bwd_dq_rows() { return kBwdWaves * 32; }
int bwd_dkdv_keys() { return 128; }

template <int D, bool CAUSAL>
static hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  const long long pairs = (long long)p.ws_stride * p.hq;
  const int ppb = 256 / (D / 8);
  const int n_kv = p.batch * p.hkv * p.n_kblocks, n_q = p.batch * p.hq * p.n_qtiles;
  // A side with no rows launches nothing: with no queries the dK/dV kernel
  // still runs and writes zeros, with no keys the dQ kernel does.
  if (pairs > 0)
    hipLaunchKernelGGL(bwd_preprocess_kernel<D>, dim3((unsigned)((pairs + ppb - 1) / ppb)),
                       dim3(256), 0, stream, p);
  if (n_kv > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(n_kv), dim3(512), 0, stream, p);
  if (n_q > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D, kBwdWaves, CAUSAL>), dim3(n_q), dim3(kBwdWaves * 64),
                       0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int head_dim, bool causal, hipStream_t stream) {
  if (head_dim == 128)
    return causal ? launch_bwd_d<128, true>(p, stream) : launch_bwd_d<128, false>(p, stream);
  return causal ? launch_bwd_d<64, true>(p, stream) : launch_bwd_d<64, false>(p, stream);
}

}  // namespace fa
