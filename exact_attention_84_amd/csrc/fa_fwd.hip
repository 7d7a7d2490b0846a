// Fused attention forward (prefill): fixed-length batches and packed
// variable-length sequences, causal or not, MHA or GQA.
//
// Work decomposition: one workgroup per (sequence, query head, tile of BR
// query rows) -- causal: a pair of tiles, n-1-i and i, of the same sequence;
// the Q tile stays in registers while K/V tiles of BC keys stream through LDS
// ("FlashAttention — IO 感知的精确注意力 kernel", section 2.3 step 4: one Q
// tile per thread block, K/V tiles streamed through on-chip memory, launched
// over (Q blocks, batch, head)).  Causal tiles stop at the diagonal, so a
// causal forward does about half the work ("推理优化 | FlashAttention 1-4
// 详解", section FlashAttention 2 的工程优化, causal lower-triangle
// skipping).  Masks are applied only on tiles that cross the diagonal or the
// end of the keys.
//
// Within a wave the key loop is software-pipelined so that the matrix core and
// the ALUs work at the same time (the GEMM/softmax overlap of the first page's
// FlashAttention 3 notes, section FlashAttention 3 的硬件特性利用, done here
// inside one wavefront): step j computes the scores of tile j, then issues the
// P V MFMAs of tile j-1 one by one with a slice of the softmax of tile j after
// each.
//
// The score variants the code-reading page lists as compile-time switches
// next to causal masking ("FlashAttention — IO 感知的精确注意力 kernel",
// section 1 capability table: sliding window, ALiBi, softcap) are further
// instances of the same pipelined body.  For query i and key j of a sequence
// (delta = Lk - Lq aligns the last query with the last key):
//   x_ij = scale <q_i, k_j>
//   x_ij = cap tanh(x_ij / cap)                      (softcap, cap > 0)
//   x_ij = x_ij - slope_h |i + delta - j|            (ALiBi, slopes given)
//   j admissible: 0 <= j < Lk, and
//     j >= i + delta - left  (left >= 0),  j <= i + delta + right (right >= 0),
//     j <= i + delta         (causal)
// The local instance visits only the key tiles that hold admissible keys of
// the workgroup's rows, so a window of w keys costs about w keys per query;
// the transform instance adds the softcap and ALiBi to every score it forms.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

// Sets to -inf every score of a 64-key tile whose key lies past the lane's
// limit.  Key kt*32 + 4 hh + c_v (c_v = (v & 3) + 8 (v >> 2)) of the tile is
// admissible for the query of lane (t, m32) when its offset from the tile's
// first key, minus 4 hh, is <= lim[t]: one compare per element.
template <int NT, int NKT>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[NKT][NT], const int (&lim)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if ((v & 3) + 8 * (v >> 2) + 32 * kt > lim[t]) s[kt][t][v] = -INFINITY;
}

// Sets to -inf every score of a 64-key tile whose key lies before the lane's
// first admissible key (a local window's left edge): key offset minus 4 hh
// below lo[t].
template <int NT, int NKT>
__device__ __forceinline__ void mask_tile_lo(f32x16 (&s)[NKT][NT], const int (&lo)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if ((v & 3) + 8 * (v >> 2) + 32 * kt < lo[t]) s[kt][t][v] = -INFINITY;
}

// Per-score transform of the ALiBi / softcap instance: the raw score s of
// query row qi and key kj becomes, in log2 units (L = log2 e),
//   y = s * scale;  y = cap * tanh(y / cap) (cap > 0);  y -= slope |qi + delta - kj|
// with tanh(x) = 1 - 2 / (exp(2x) + 1) from one exp2 and one hardware
// reciprocal (each within an ulp or so; exp2 -> inf gives tanh = 1).  The
// constants arrive folded: k = scale L without a cap, 2 scale L / cap with
// one; cap_l = cap L (0: no cap); slope_l = slope L.  rel[t] is
// qi + delta - 4 hh - k0 for the lane's row of group t and the tile's first
// key k0, so that the distance of element (kt, v) is |rel - 32 kt - c_v|.
struct ScoreXf {
  float k, cap_l, slope_l;
};
template <int NT, int NKT>
__device__ __forceinline__ void transform_tile(f32x16 (&s)[NKT][NT], const ScoreXf& x,
                                               const int (&rel)[NT]) {
  if (x.cap_l > 0.f) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float e = fast_exp2(s[kt][t][v] * x.k);
          s[kt][t][v] = fmaf(-2.f * x.cap_l, __builtin_amdgcn_rcpf(e + 1.f), x.cap_l);
        }
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kt][t][v] *= x.k;
  }
  if (x.slope_l != 0.f) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float r = static_cast<float>(rel[t]);  // exact: |rel| < 2^24
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float c = static_cast<float>(32 * kt + (v & 3) + 8 * (v >> 2));
          s[kt][t][v] = fmaf(-x.slope_l, fabsf(r - c), s[kt][t][v]);
        }
    }
  }
}

// One steady-state step of a wave owning NT groups of 32 query rows, 64-key
// tiles:
//   s      = Q K_j^T            (D/8 K fragments, NT MFMAs each)
//   O     += P_{j-1} V_{j-1}    (D/8 V fragments, NT MFMAs each)
//   probabilities of s (tile j) -> pout
// The P V MFMAs do not depend on the new scores, so each of them is followed
// by a slice of the exponentials of s (sched_barrier fences keep that order):
// the wave keeps issuing ALU instructions while the matrix core works.
//
// The probabilities are first formed against each row's current reference r,
// with no row maximum: p = 2^(s c - r).  Every p of a lane is at most the
// lane's sum of them, so when no lane's sum exceeds kSumCap (and none is inf
// or NaN: a row still at r = -inf gives inf or NaN) the reference may stay
// and the step is done (alpha = 1).  Otherwise the tile's scores, kept
// unchanged, go through the row-maximum path of softmax_probs, which moves
// the references.  Either way O and l are accumulated relative to the same
// r, so the result is the same up to rounding.  Returns whether a row moved
// its reference (alpha then holds the rescale factors).  A tile that crosses
// the end of the keys or the diagonal is masked first (`masked`, uniform over
// the wave; limits as in mask_tile).
template <int D, int NT, bool LOCAL, bool XF>
__device__ __forceinline__ bool steady_step(WaveState<D, NT>& st, const char* __restrict__ k_cur,
                                            const char* __restrict__ v_prev, const LdsRead<D>& rd,
                                            const bf16x8 (&pin)[2][NT][2],
                                            bf16x8 (&pout)[2][NT][2], float (&alpha)[NT],
                                            float c, bool masked, const int (&lim)[NT],
                                            const int (&lo)[NT], const ScoreXf& xf,
                                            const int (&rel)[NT]) {
  constexpr int DT = D / 32;
  constexpr int SLOTS = D / 8;                  // V fragments per step
  constexpr int LEAD = 2;                       // P V MFMAs before the first slice
  constexpr int NE = 32 * NT;                   // probabilities per lane
  constexpr int EXP_SLOTS = SLOTS - LEAD;
  static_assert(4 * DT == SLOTS, "slot bookkeeping");

  f32x16 s[2][NT];
  scores_tile<D, NT, 2>(s, k_cur, rd, st.qf);
  if constexpr (XF) transform_tile<NT, 2>(s, xf, rel);
  if (masked) {
    mask_tile<NT, 2>(s, lim);
    if constexpr (LOCAL) mask_tile_lo<NT, 2>(s, lo);
  }

  float rs[NT];
  uint32_t pk[NT][16];
#pragma unroll
  for (int t = 0; t < NT; ++t) rs[t] = 0.f;
  bf16x8 va = rd.v(v_prev, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int pkt = i / (2 * DT), pu = (i / DT) & 1, pdt = i % DT;
    const bf16x8 vcur = va;
    if (i + 1 < SLOTS) {
      const int n = i + 1;
      va = rd.v(v_prev, n / (2 * DT), (n / DT) & 1, n % DT);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
      st.o[t][pdt] = mfma_32x32x16(vcur, pin[pkt][t][pu], st.o[t][pdt]);
    __builtin_amdgcn_sched_barrier(0);
    if (i >= LEAD) {
      // pairs of probabilities g0 .. g1-1 of the lane's NE / 2, spread evenly
      // over the slots; the scores stay in place for the row-maximum path
      const int g0 = (i - LEAD) * (NE / 2) / EXP_SLOTS;
      const int g1 = (i - LEAD + 1) * (NE / 2) / EXP_SLOTS;
#pragma unroll
      for (int g = g0; g < g1; ++g) {
        const int t = g >> 4, e = 2 * (g & 15);
        const float p0 = fast_exp2(fmaf(s[e >> 4][t][e & 15], c, -st.mc[t]));
        const float p1 = fast_exp2(fmaf(s[e >> 4][t][(e + 1) & 15], c, -st.mc[t]));
        rs[t] += p0;
        rs[t] += p1;
        pk[t][e >> 1] = pack_bf16x2(p0, p1);
        // keep the conversion in this slice (it would otherwise sink to its
        // use in the next step)
        asm volatile("" ::"v"(pk[t][e >> 1]));
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(rs[t]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  bool ok = true;
#pragma unroll
  for (int t = 0; t < NT; ++t) ok = ok && (rs[t] <= kSumCap);
  if (__builtin_expect(__all(ok), 1)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4 w = {pk[t][8 * kt + 4 * u], pk[t][8 * kt + 4 * u + 1],
                           pk[t][8 * kt + 4 * u + 2], pk[t][8 * kt + 4 * u + 3]};
          pout[kt][t][u] = __builtin_bit_cast(bf16x8, w);
        }
      st.l[t] += rs[t];
      alpha[t] = 1.f;
    }
    return false;
  }
  // some row outgrew its reference (or has none yet): the row-maximum path
  return softmax_probs<D, NT, 2>(st, s, pout, alpha, c);
}

// The steady step with the row maximum first (the transform instance's):
// each P V MFMA is followed by a slice of the softmax of s, the row maxima
// and new references in the first two slices, then the exponentials against
// the new references.  ALiBi raises the scores of every tile nearer the
// diagonal, so its references move on most tiles; forming the maxima first
// costs less there than forming the probabilities twice.  Returns whether a
// row moved its reference (alpha then holds the rescale factors).
template <int D, int NT, bool LOCAL, bool XF>
__device__ __forceinline__ bool steady_step_max_first(
    WaveState<D, NT>& st, const char* __restrict__ k_cur, const char* __restrict__ v_prev,
    const LdsRead<D>& rd, const bf16x8 (&pin)[2][NT][2], bf16x8 (&pout)[2][NT][2],
    float (&alpha)[NT], float c, bool masked, const int (&lim)[NT], const int (&lo)[NT],
    const ScoreXf& xf, const int (&rel)[NT]) {
  constexpr int DT = D / 32;
  constexpr int SLOTS = D / 8;                  // V fragments per step
  constexpr int LEAD = 2;                       // P V MFMAs before the first slice
  constexpr int NE = 32 * NT;                   // probabilities per lane
  constexpr int EXP_SLOTS = SLOTS - LEAD - 2;   // two slots hold the row maxima
  constexpr int PER = (NE + EXP_SLOTS - 1) / EXP_SLOTS;
  static_assert(4 * DT == SLOTS, "slot bookkeeping");

  f32x16 s[2][NT];
  scores_tile<D, NT, 2>(s, k_cur, rd, st.qf);
  if constexpr (XF) transform_tile<NT, 2>(s, xf, rel);
  if (masked) {
    mask_tile<NT, 2>(s, lim);
    if constexpr (LOCAL) mask_tile_lo<NT, 2>(s, lo);
  }

  float mx[NT], msub[NT], rs[NT], mref[NT];
  uint32_t pk[NT][16];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    mx[t] = -INFINITY;
    rs[t] = 0.f;
  }
  bf16x8 va = rd.v(v_prev, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int pkt = i / (2 * DT), pu = (i / DT) & 1, pdt = i % DT;
    const bf16x8 vcur = va;
    if (i + 1 < SLOTS) {
      const int n = i + 1;
      va = rd.v(v_prev, n / (2 * DT), (n / DT) & 1, n % DT);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
      st.o[t][pdt] = mfma_32x32x16(vcur, pin[pkt][t][pu], st.o[t][pdt]);
    __builtin_amdgcn_sched_barrier(0);
    if (i == LEAD) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx[t] = fmaxf(mx[t], s[0][t][v]);
    } else if (i == LEAD + 1) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int v = 0; v < 16; ++v) mx[t] = fmaxf(mx[t], s[1][t][v]);
        const float mx_c = halfwave_max(mx[t]) * c;
        mref[t] = (mx_c > st.mc[t] + kRescaleTau) ? mx_c : st.mc[t];
        msub[t] = (mref[t] == -INFINITY) ? 0.f : mref[t];
        alpha[t] = fast_exp2(st.mc[t] - msub[t]);
      }
    } else if (i > LEAD + 1) {
      const int e0 = (i - LEAD - 2) * PER;
#pragma unroll
      for (int g = e0; g < e0 + PER && g < NE; ++g) {
        const int t = g >> 5, e = g & 31;
        const float pe = fast_exp2(fmaf(s[e >> 4][t][e & 15], c, -msub[t]));
        s[e >> 4][t][e & 15] = pe;
        rs[t] += pe;
        if (e & 1) {
          pk[t][e >> 1] = pack_bf16x2(s[e >> 4][t][(e - 1) & 15], pe);
          // keep the conversion in this slice (it would otherwise sink to
          // its use in the next step)
          asm volatile("" ::"v"(pk[t][e >> 1]));
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(rs[t]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  bool moved = false;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 w = {pk[t][8 * kt + 4 * u], pk[t][8 * kt + 4 * u + 1],
                         pk[t][8 * kt + 4 * u + 2], pk[t][8 * kt + 4 * u + 3]};
        pout[kt][t][u] = __builtin_bit_cast(bf16x8, w);
      }
    st.l[t] = fmaf(alpha[t], st.l[t], rs[t]);
    moved |= mref[t] != st.mc[t];
    st.mc[t] = mref[t];
  }
  return moved;
}

// Two waves per SIMD (256 registers each) when a wave owns 32 query rows, so
// that one wave's MFMAs overlap the other's softmax arithmetic.  NW is 4 or 8
// (fwd_waves); PAIR runs two causal query tiles per workgroup.
//
// LOCAL adds a local window: query i sees keys i + delta - left .. i + delta +
// right (a negative bound open), visited from the workgroup's first window
// tile on; tiles that cross a row's left edge are masked like edge tiles.
template <int D, int NW, int NT, bool CAUSAL, bool PAIR, bool LOCAL, bool XF = false>
__device__ __forceinline__ void fwd_body(const FwdParams& p, int win_left, int win_right,
                                         const ScoreXf& xf = ScoreXf{}) {
  constexpr int BC = 64;
  constexpr int NKT = BC / 32;
  constexpr int BR = NW * 32 * NT;
  constexpr int TILE_BYTES = BC * D * 2;
  // Two stages of K and V: the next tiles stream in while these are used.
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index is the same for all lanes; saying so keeps every quantity
  // derived from it (this wave's rows, its tile count, the loop conditions) in
  // scalar registers and the control flow wave-uniform.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m32 = lane & 31, hh = lane >> 5;

  // ---- work item: (sequence b, kv head, query head in group, query tile) ----
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
  // One query tile, as a function of its index, inlined at its one call site.
  auto run_tile = [&](const int qt) __attribute__((always_inline)) {
  const int q0 = qt * BR;

  const int delta = Lk - Lq;  // bottom-right causal offset
  // LOCAL: right edge offset of the window (causal caps it at 0; -1 = none)
  const int right = !LOCAL ? -1 : (CAUSAL ? (win_right < 0 ? 0 : min(win_right, 0)) : win_right);
  // first key of query i's window (LOCAL with a left edge), else 0
  auto key_lo = [&](int i) { return (LOCAL && win_left >= 0) ? max(0, i + delta - win_left) : 0; };
  // Tiles kt0 .. kt0 + n_kt - 1 are visited; step j works on tile kt0 + j.
  const int kt0 = LOCAL ? min(key_lo(q0), Lk) / BC : 0;
  int n_kt = (Lk + BC - 1) / BC;
  if (!LOCAL && CAUSAL) {
    const int last_key = min(Lk - 1, q0 + BR - 1 + delta);
    n_kt = last_key < 0 ? 0 : min(n_kt, last_key / BC + 1);
  }
  if (LOCAL && right >= 0) {
    const int last_key = min(Lk - 1, q0 + BR - 1 + delta + right);
    n_kt = last_key < 0 ? 0 : min(n_kt, last_key / BC + 1);
  }
  if constexpr (LOCAL) n_kt = max(0, n_kt - kt0);
  const int qw0 = q0 + wave * 32 * NT;
  const bool wave_active = qw0 < Lq;
  const int wave_last_key =
      !LOCAL ? (CAUSAL ? min(Lk - 1, qw0 + 32 * NT - 1 + delta) : Lk - 1)
             : (right >= 0 ? min(Lk - 1, qw0 + 32 * NT - 1 + delta + right) : Lk - 1);
  // Key tiles this wave needs (causal: up to its own diagonal).
  const int wn = !LOCAL ? ((wave_active && wave_last_key >= 0) ? min(n_kt, wave_last_key / BC + 1) : 0)
                        : ((wave_active && wave_last_key >= kt0 * BC)
                               ? min(n_kt, wave_last_key / BC + 1 - kt0) : 0);

  const size_t q_stride = (size_t)p.hq * D;
  const size_t kv_stride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + (size_t)k_start * kv_stride + (size_t)kvh * D;
  const uint16_t* vbase = p.v + (size_t)k_start * kv_stride + (size_t)kvh * D;

  TileDMA<D, BC, NW> dma;
  dma.init(kv_stride, wave, lane);
  LdsRead<D> rd;
  rd.init(lane);
  if (n_kt > 0) dma.issue(kbase, kv_stride, kt0 * BC, Lk - 1, k_lds0, wave, lane);

  WaveState<D, NT> st;
  st.init();
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int qi = qw0 + t * 32 + m32;
    const uint16_t* qp = p.q + (size_t)(q_start + qi) * q_stride + (size_t)h * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qi < Lq) raw = *reinterpret_cast<const u32x4*>(qp + 16 * s);
      st.qf[t][s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // Score tile j needs a mask when it crosses the end of the keys or (causal)
  // this wave's diagonal; both only grow with j.
  auto edge_tile = [&](int j) {
    const int k0 = (kt0 + j) * BC;
    if constexpr (LOCAL)
      return (k0 + BC > Lk) || (right >= 0 && k0 + BC - 1 > qw0 + delta + right) ||
             (k0 < key_lo(qw0 + 32 * NT - 1));
    return (k0 + BC > Lk) || (CAUSAL && k0 + BC - 1 > qw0 + delta);
  };
  // Last admissible key of each of this lane's query rows, min(Lk - 1,
  // qi + Lk - Lq) causal or Lk - 1, minus 4 hh (the lane's key offset in a
  // tile); tile j masks against row_lim - j * BC.
  int row_lim[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int qi = qw0 + t * 32 + m32;
    if constexpr (LOCAL)
      row_lim[t] = (right >= 0 ? min(Lk - 1, qi + delta + right) : Lk - 1) - 4 * hh;
    else
      row_lim[t] = (CAUSAL ? min(Lk - 1, qi + delta) : Lk - 1) - 4 * hh;
  }
  // LOCAL: first admissible key of each of this lane's rows, minus 4 hh
  int row_lo[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) row_lo[t] = key_lo(qw0 + t * 32 + m32) - 4 * hh;
  // XF: the lane's aligned diagonal position, minus 4 hh (ALiBi distances)
  int row_rel[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) row_rel[t] = qw0 + t * 32 + m32 + delta - 4 * hh;
  // Step j: K_j and V_{j-1} are in LDS; K_{j+1} and V_j start streaming into
  // the stages that K_{j-1} and V_{j-2} used.
  // The loads are asm, issued with no branch per instruction (the tile's rows
  // clamped to the last key); wait_dma and the barrier order them.
  constexpr int PW = decltype(dma)::PER_WAVE;
  const uint32_t kv_row_bytes = 2u * (uint32_t)kv_stride;
  auto stage = [&](int j) {
    wait_dma();       // this wave's share of K_j and V_{j-1} has landed
    __syncthreads();  // everyone's has, and everyone is done with K_{j-1}, V_{j-2}
    if (j + 1 < n_kt) {
      const auto src = decltype(dma)::src(kbase, kv_stride, (kt0 + j + 1) * BC, Lk - 1);
      const uint32_t at = lds_address((j & 1) ? k_lds0 : k_lds1);
      auto one = [&](auto nc) {
        dma.template issue_one<decltype(nc)::value>(src, kv_row_bytes, at, wave);
      };
      static_for<PW>(one);
    }
    if (j < n_kt) {
      const auto src = decltype(dma)::src(vbase, kv_stride, (kt0 + j) * BC, Lk - 1);
      const uint32_t at = lds_address((j & 1) ? v_lds1 : v_lds0);
      auto one = [&](auto nc) {
        dma.template issue_one<decltype(nc)::value>(src, kv_row_bytes, at, wave);
      };
      static_for<PW>(one);
    }
  };

  // The O rescale of tile j (alpha_j, when some row moved its reference) must
  // land after P_{j-1} V_{j-1} and before P_j V_j: it is applied at the top of
  // step j+1.  p_a / p_b hold the probabilities of tiles j-1 and j.
  bf16x8 p_a[NKT][NT][2], p_b[NKT][NT][2];
  float alpha[NT];
  bool moved = false;

  // One step done phase by phase (first tile, masked tiles, the final P V).
  auto general_step = [&](int j) {
    stage(j);
    const char* k_cur = (j & 1) ? k_lds1 : k_lds0;
    const char* v_prev = (j & 1) ? v_lds0 : v_lds1;
    if (j >= 1 && j <= wn) {
      if (__any(moved)) rescale_o<D, NT>(st, alpha);
      pv_tile<D, NT, NKT>(st, v_prev, rd, p_a);
    }
    if (j < wn) {
      f32x16 s[NKT][NT];
      scores_tile<D, NT, NKT, false>(s, k_cur, rd, st.qf);
      if constexpr (XF) {
        int rel[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) rel[t] = row_rel[t] - (kt0 + j) * BC;
        transform_tile<NT, NKT>(s, xf, rel);
      }
      if (edge_tile(j)) {
        int lim[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) lim[t] = row_lim[t] - (kt0 + j) * BC;
        mask_tile<NT, NKT>(s, lim);
        if constexpr (LOCAL) {
          int lo[NT];
#pragma unroll
          for (int t = 0; t < NT; ++t) lo[t] = row_lo[t] - (kt0 + j) * BC;
          mask_tile_lo<NT, NKT>(s, lo);
        }
      }
      moved = softmax_probs<D, NT, NKT>(st, s, p_a, alpha, p.c);
    }
  };

  int j = 0;
  // Steady steps: 1 <= j < wn, each one the scores of tile j and the P V of
  // tile j-1, masked when tile j crosses the end of the keys or this wave's
  // diagonal.  Unrolled by two so that the LDS stages and the probability
  // registers swap statically.  Step 0 (no P V yet), the final P V and the
  // steps where this wave has no tile left (the workgroup's other waves
  // still do) take the generic path.
  auto steady = [&](int jj, const char* k_cur, const char* v_prev, const bf16x8 (&pin)[NKT][NT][2],
                    bf16x8 (&pout)[NKT][NT][2]) {
    stage(jj);
    if (__any(moved)) rescale_o<D, NT>(st, alpha);
    int lim[NT], lo[NT], rel[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      lim[t] = row_lim[t] - (kt0 + jj) * BC;
      lo[t] = row_lo[t] - (kt0 + jj) * BC;
      rel[t] = row_rel[t] - (kt0 + jj) * BC;
      // opaque per step: otherwise the compiler carries every element's
      // mask threshold from step to step, paying for it on unmasked steps
      asm volatile("" : "+v"(lim[t]), "+v"(lo[t]));
    }
    if constexpr (XF)
      moved = steady_step_max_first<D, NT, LOCAL, XF>(st, k_cur, v_prev, rd, pin, pout, alpha,
                                                      p.c, edge_tile(jj), lim, lo, xf, rel);
    else
      moved = steady_step<D, NT, LOCAL, XF>(st, k_cur, v_prev, rd, pin, pout, alpha, p.c,
                                            edge_tile(jj), lim, lo, xf, rel);
  };
  if (wn > 1) {
    general_step(0);  // softmax of S_0 -> p_a
    // the Q loads are known complete from here on: the compiler then puts no
    // waits for them inside the loop, where the counter also counts the asm
    // tile loads (step 1 waits for those anyway)
    vm_drain();
    j = 1;
#pragma clang loop unroll(disable)
    while (j < wn) {
      // odd j: K_j in stage 1, V_{j-1} in stage 0, P_{j-1} in p_a
      steady(j, k_lds1, v_lds0, p_a, p_b);
      ++j;
      if (j >= wn) {
        // the generic step expects P_{j-1} in p_a
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int u = 0; u < 2; ++u) p_a[kt][t][u] = p_b[kt][t][u];
        break;
      }
      // even j: K_j in stage 0, V_{j-1} in stage 1, P_{j-1} in p_b
      steady(j, k_lds0, v_lds1, p_b, p_a);
      ++j;
    }
  }
#pragma clang loop unroll(disable)
  for (; j <= n_kt; ++j) general_step(j);

  // ---- epilogue: O / l, LSE = ln 2 * (r c + log2 l) ----
  // O goes out through this wave's 8 KB of the K/V stages, free once every
  // wave is past its last P V, as whole 16-byte chunks of row runs
  static_assert(NW == 4, "one K/V stage buffer per wave holds its output rows");
  __syncthreads();
  char* const stg = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
  const size_t esz = p.o_f32 ? 4 : 2;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lt = halfwave_sum(st.l[t]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (st.mc[t] + __log2f(lt)) * kLn2 : -INFINITY;
    const int qi = qw0 + t * 32 + m32;
    if (qi < Lq && hh == 0) p.lse[(size_t)(q_start + qi) * p.hq + h] = lse;
    const int r0 = qw0 + t * 32;  // the row group's first row
    store_rows_lds<D>(st.o[t], inv,
                      reinterpret_cast<char*>(p.o) + ((size_t)(q_start + r0) * p.hq + h) * D * esz,
                      (size_t)p.hq * D * esz, Lq - r0, p.o_f32 != 0, stg, lane);
  }
  };  // run_tile

  if constexpr (PAIR) {
    // Causal: under the diagonal tile i of a sequence with n tiles costs about
    // i + 1 key tiles, so tile n-1-i (heaviest first) is paired with tile i
    // and every workgroup of the sequence gets n + 1 key tiles of work.  n is
    // this sequence's own tile count, so packed sequences pair the same way.
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

template <int D, int NW, int NT, bool CAUSAL, bool PAIR>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 2 : 1)))
void fwd_kernel(const FwdParams p) {
  fwd_body<D, NW, NT, CAUSAL, PAIR, false>(p, -1, -1);
}

// A local (sliding) window on the same pipelined path: 4-wave workgroups, no
// tile pairing (a window makes every query tile cost about the same).
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_local_kernel(const FwdParams p, int win_left, int win_right) {
  fwd_body<D, NW, kFwdNT, CAUSAL, false, true>(p, win_left, win_right);
}

// The local instance with the ALiBi / softcap transform: the slope is per
// (sequence, query head), read from alibi[b * alibi_stride + h].
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_xf_kernel(const FwdParams p, int win_left, int win_right, float scale, float cap,
                   const float* alibi, int alibi_stride) {
  // the slope of this workgroup's (sequence, head), found as fwd_body finds them
  const int item = xcd_remap(blockIdx.x, p.total, p.group * p.n_items);
  int rest = item / p.n_items;
  const int hg = rest % p.group;
  rest /= p.group;
  const int kvh = rest % p.hkv;
  const int b = rest / p.hkv;
  const float slope = alibi ? alibi[(size_t)b * alibi_stride + kvh * p.group + hg] : 0.f;
  ScoreXf xf;
  xf.k = cap > 0.f ? 2.f * scale * kLog2e / cap : scale * kLog2e;
  xf.cap_l = cap * kLog2e;
  xf.slope_l = slope * kLog2e;
  fwd_body<D, NW, kFwdNT, CAUSAL, false, true, true>(p, win_left, win_right, xf);
}

// Explicit instantiations: every kernel the dispatcher can launch is emitted
// on both the device and the host side.
template __global__ void fwd_kernel<64, 4, kFwdNT, false, false>(const FwdParams);
template __global__ void fwd_kernel<64, 4, kFwdNT, true, true>(const FwdParams);
template __global__ void fwd_local_kernel<128, 4, false>(const FwdParams, int, int);
template __global__ void fwd_local_kernel<128, 4, true>(const FwdParams, int, int);
template __global__ void fwd_local_kernel<64, 4, false>(const FwdParams, int, int);
template __global__ void fwd_local_kernel<64, 4, true>(const FwdParams, int, int);
template __global__ void fwd_xf_kernel<128, 4, false>(const FwdParams, int, int, float, float,
                                                      const float*, int);
template __global__ void fwd_xf_kernel<128, 4, true>(const FwdParams, int, int, float, float,
                                                     const float*, int);
template __global__ void fwd_xf_kernel<64, 4, false>(const FwdParams, int, int, float, float,
                                                     const float*, int);
template __global__ void fwd_xf_kernel<64, 4, true>(const FwdParams, int, int, float, float,
                                                    const float*, int);

template <int D, int NW, int NT, bool CAUSAL, bool PAIR>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_kernel<D, NW, NT, CAUSAL, PAIR>), dim3(p.total), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

// Kernel and workgroup shape of a call.  Plain attention at head dim 128,
// causal or not, runs the 64-row-wave kernel: 4 waves (256 rows) for
// fixed-length batches of at least 1024 queries, else 2 (128 rows: less
// padding and more workgroups for short or packed sequences).  Causal calls
// there pair heavy and light query tiles as the 32-row kernel does; at one
// wave per SIMD the waves that reach their diagonal first leave their SIMDs
// idle, and still the kernel measured 3 % faster than the 32-row one on the
// fixed-length causal workloads and level on the packed one.  The 32-row
// kernels (head dim 64, the score variants and FP8) take 4 waves (128 rows),
// so that two workgroups share a compute unit and the two waves on each SIMD
// come from different workgroups: not held in step by one workgroup's
// barriers, one wave's exponentials run beside the other's matrix products.
// For FP8 that measured 9 % faster than 8-wave workgroups on the
// B=4 H=16 N=2048 workload (8 waves halve the K/V loads per query).
FwdPlan fwd_plan(FwdKind kind, int head_dim, bool causal, bool varlen, int seqlen_q) {
  if (kind == FwdKind::Plain && head_dim == 128) {
    const int w = (!varlen && seqlen_q >= 1024) ? 4 : 2;
    return {w, w * 64, 1};
  }
  return {4, 4 * 32 * kFwdNT, 0};
}

template <int D, int NW>
static hipError_t launch_dw(const FwdParams& p, bool causal, hipStream_t stream) {
  return causal ? launch_one<D, NW, kFwdNT, true, true>(p, stream)
                : launch_one<D, NW, kFwdNT, false, false>(p, stream);
}

hipError_t launch_fwd_local(const FwdParams& p, int head_dim, bool causal, int win_left,
                            int win_right, hipStream_t stream) {
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(p.total), dim3(256), 0, stream, p, win_left, win_right);
    return hipGetLastError();
  };
  if (head_dim == 128)
    return causal ? go(fwd_local_kernel<128, 4, true>) : go(fwd_local_kernel<128, 4, false>);
  return causal ? go(fwd_local_kernel<64, 4, true>) : go(fwd_local_kernel<64, 4, false>);
}

hipError_t launch_fwd_xf(const FwdParams& p, int head_dim, bool causal, int win_left,
                         int win_right, float scale, float cap, const float* alibi,
                         int alibi_stride, hipStream_t stream) {
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(p.total), dim3(256), 0, stream, p, win_left, win_right, scale,
                       cap, alibi, alibi_stride);
    return hipGetLastError();
  };
  if (head_dim == 128)
    return causal ? go(fwd_xf_kernel<128, 4, true>) : go(fwd_xf_kernel<128, 4, false>);
  return causal ? go(fwd_xf_kernel<64, 4, true>) : go(fwd_xf_kernel<64, 4, false>);
}

// Plain attention: head dim 64 on the 32-row kernel, head dim 128 on the
// 64-row kernel (fwd_plan sets p.wide for every such call).
hipError_t launch_fwd(const FwdParams& p, int head_dim, bool causal, hipStream_t stream) {
  if (head_dim == 64) return launch_dw<64, 4>(p, causal, stream);
  if (p.wide) return launch_fwd_wide(p, causal, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
