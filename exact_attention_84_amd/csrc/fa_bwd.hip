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
#include "fa_device.hpp"
#include "fa_internal.hpp"

#ifndef FA_DKDV_WPE
#define FA_DKDV_WPE 1
#endif

namespace fa {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// D[h][r] = sum_d dO[r][h][d] O[r][h][d] and LSE[r][h] log2(e), one group of
// D/8 lanes per (row, head).
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
  if (valid && sub == 0) {
    const size_t w = (size_t)h * p.ws_stride + r;
    p.dsum[w] = acc;
    p.lse2[w] = p.lse[(size_t)r * p.hq + h] * kLog2e;  // -inf stays -inf
  }
}

// Stores a wave's 32 columns (lanes) x D rows accumulator, scaled, as rows of
// `out` ([row][head][d]): lane m32 writes row `row`, head dims dt*32 + 8g +
// 4hh + 0..3 from registers 4g..4g+3 of block dt.
template <int D>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[D / 32], float scale, void* out,
                                           size_t row_off, int f32, int hh) {
  if (f32) {
    float* op = reinterpret_cast<float*>(out) + row_off + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 w = {acc[dt][4 * g] * scale, acc[dt][4 * g + 1] * scale,
                         acc[dt][4 * g + 2] * scale, acc[dt][4 * g + 3] * scale};
        *reinterpret_cast<f32x4*>(op + dt * 32 + 8 * g) = w;
      }
  } else {
    uint16_t* op = reinterpret_cast<uint16_t*>(out) + row_off + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = {pack_bf16x2(acc[dt][4 * g] * scale, acc[dt][4 * g + 1] * scale),
                         pack_bf16x2(acc[dt][4 * g + 2] * scale, acc[dt][4 * g + 3] * scale)};
        *reinterpret_cast<u32x2*>(op + dt * 32 + 8 * g) = w;
      }
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
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m32 = lane & 31, hh = lane >> 5;

  const int total = p.batch * p.hq * p.n_qtiles;
  const int item = xcd_remap(blockIdx.x, total, p.group * p.n_qtiles);
  const int it = item % p.n_qtiles;
  int rest = item / p.n_qtiles;
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
  const int qt = CAUSAL ? p.n_qtiles - 1 - it : it;  // causal: heaviest tiles first
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
  if (n_kt > 0) {
    dma.issue(kbase, kv_stride, 0, Lk - 1, k_lds0, wave, lane);
    dma.issue(vbase, kv_stride, 0, Lk - 1, v_lds0, wave, lane);
  }
  const int wave_last_key = CAUSAL ? min(Lk - 1, qw0 + 31 + delta) : Lk - 1;

#pragma clang loop unroll(disable)
  for (int j = 0; j < n_kt; ++j) {
    const char* kc = (j & 1) ? k_lds1 : k_lds0;
    const char* vc = (j & 1) ? v_lds1 : v_lds0;
    wait_dma();
    __syncthreads();  // K_j, V_j have landed; everyone is done with the other stage
    if (j + 1 < n_kt) {
      dma.issue(kbase, kv_stride, (j + 1) * BC, Lk - 1, (j & 1) ? k_lds0 : k_lds1, wave, lane);
      dma.issue(vbase, kv_stride, (j + 1) * BC, Lk - 1, (j & 1) ? v_lds0 : v_lds1, wave, lane);
    }
    if (qw0 >= Lq) continue;  // this wave has no rows (uniform)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int ksub = j * BC + 32 * kt;
      if (ksub > wave_last_key) break;  // past this wave's keys (uniform)
      f32x16 s[1][1], dp[1][1];
      scores_tile<D, 1, 1>(s, kc + kt * 64 * D, rd, st.qf);
      scores_tile<D, 1, 1>(dp, vc + kt * 64 * D, rd, dof);
      const int lim = row_lim - ksub;
      float ds[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const bool ok = row_ok && (v & 3) + 8 * (v >> 2) <= lim;
        const float pe = ok ? fast_exp2(fmaf(s[0][0][v], p.c, -lse2)) : 0.f;
        ds[v] = ok ? pe * (dp[0][0][v] - dsum) : 0.f;
      }
      bf16x8 dsb[1][1][2];
      dsb[0][0][0] = pack_bf16x8(ds);
      dsb[0][0][1] = pack_bf16x8(ds + 8);
      pv_tile<D, 1, 1>(st, kc + kt * 64 * D, rd, dsb);  // dQ^T += K^T dS^T
    }
  }
  if (row_ok)
    store_rows<D>(st.o[0], p.scale, p.dq, ((size_t)(q_start + qi) * p.hq + h) * D, p.g_f32, hh);
}

// ---------------------------------------------------------------------------
// dK, dV: each wave owns 32 keys (one per lane column).  Per 32-query
// sub-tile of the streamed Q / dO tiles it forms S = Q K^T and dP = dO V^T
// (rows = queries), P and dS in registers with the query rows' LSE and D,
// then dV^T += dO^T P and dK^T += Q^T dS.  The rows' LSE log2(e) and D ride
// along with each Q / dO tile into LDS, so the inner loop reads no global
// memory.
// ---------------------------------------------------------------------------
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(FA_DKDV_WPE)))
void bwd_dkdv_kernel(const BwdParams p) {
  constexpr int BQ = 64;
  constexpr int BK = NW * 32;
  constexpr int TILE = BQ * D * 2;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(1024))) char q_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) char q_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) char do_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) char do_lds1[TILE];
  // per stage: LSE log2(e) of the tile's 64 rows, then their D (the DMA
  // instruction fills 1 KB; the second half repeats the first)
  __shared__ __attribute__((aligned(1024))) float st_lds[2][256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m32 = lane & 31, hh = lane >> 5;

  const int total = p.batch * p.hkv * p.n_kblocks;
  const int item = xcd_remap(blockIdx.x, total, p.n_kblocks);
  const int kblk = item % p.n_kblocks;
  const int rest = item / p.n_kblocks;
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
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + m32;
  const bool key_ok = key < Lk;

  const size_t q_stride = (size_t)p.hq * D;
  const size_t kv_stride = (size_t)p.hkv * D;
  // this lane's key row of K and V (zeros past the end: their gradients are
  // accumulated but never stored)
  bf16x8 kf[1][KS], vf[1][KS];
  {
    const size_t off = (size_t)(k_start + key) * kv_stride + (size_t)kvh * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 rk = {0u, 0u, 0u, 0u}, rv = {0u, 0u, 0u, 0u};
      if (key_ok) {
        rk = *reinterpret_cast<const u32x4*>(p.k + off + 16 * s);
        rv = *reinterpret_cast<const u32x4*>(p.v + off + 16 * s);
      }
      kf[0][s] = __builtin_bit_cast(bf16x8, rk);
      vf[0][s] = __builtin_bit_cast(bf16x8, rv);
    }
  }
  WaveState<D, 1> sk, sv;  // o: dK^T and dV^T accumulators
  sk.init();
  sv.init();

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
  auto issue = [&](int step, int stage) {
    const int hg = step / per_head, q0 = (qt0 + step % per_head) * BQ;
    const int h = p.group * kvh + hg;
    const size_t head = (size_t)h * D;
    const uint16_t* qb = p.q + (size_t)q_start * q_stride + head;
    const uint16_t* db = p.dout + (size_t)q_start * q_stride + head;
    dma.issue(qb, q_stride, q0, Lq - 1, stage ? q_lds1 : q_lds0, wave, lane);
    dma.issue(db, q_stride, q0, Lq - 1, stage ? do_lds1 : do_lds0, wave, lane);
    if (wave == 0) {
      // 16 lanes x 16 bytes per statistic; the row base is clamped so the
      // 64-row read stays inside the workspace (its 64 rows of padding)
      const int r0 = min(q_start + q0, p.ws_stride - BQ);
      const float* src = ((lane & 16) ? p.dsum : p.lse2) + (size_t)h * p.ws_stride + r0 +
                         4 * (lane & 15);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)st_lds[stage], 16, 0, 0);
    }
  };
  if (n_steps > 0) issue(0, 0);

#pragma clang loop unroll(disable)
  for (int step = 0; step < n_steps; ++step) {
    const int stage = step & 1;
    const char* qc = stage ? q_lds1 : q_lds0;
    const char* dc = stage ? do_lds1 : do_lds0;
    const float* stl = st_lds[stage];
    wait_dma();
    __syncthreads();  // this tile has landed; everyone is done with the other stage
    if (step + 1 < n_steps) issue(step + 1, stage ^ 1);
    if (kw0 >= Lk) continue;  // this wave has no keys (uniform)
    const int q0 = (qt0 + step % per_head) * BQ;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int qsub = q0 + 32 * kt;
      if (qsub >= Lq) break;                            // past the queries (uniform)
      if (CAUSAL && kw0 > qsub + 31 + delta) continue;  // every key above the diagonal
      f32x16 s[1][1], dp[1][1];
      scores_tile<D, 1, 1>(s, qc + kt * 64 * D, rd, kf);   // S = Q K^T
      scores_tile<D, 1, 1>(dp, dc + kt * 64 * D, rd, vf);  // dP = dO V^T
      // the lane's rows are qsub + 8 g + 4 hh + 0..3 for register group g
      const bool full = qsub + 31 < lq_eff && (!CAUSAL || kw0 + 31 <= qsub + delta);
      const int lo = key - delta - qsub - 4 * hh;  // first admissible row offset (causal)
      const int hi = lq_eff - 1 - qsub - 4 * hh;   // last row offset with data
      float pe[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(stl + 32 * kt + 8 * g + 4 * hh);
        const f32x4 dd = *reinterpret_cast<const f32x4*>(stl + 64 + 32 * kt + 8 * g + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * g + e;
          const float pv = fast_exp2(fmaf(s[0][0][v], p.c, -l2[e]));
          const float dv = pv * (dp[0][0][v] - dd[e]);
          const int r = 8 * g + e;
          const bool ok = full || (r <= hi && (!CAUSAL || r >= lo));
          pe[v] = ok ? pv : 0.f;
          ds[v] = ok ? dv : 0.f;
        }
      }
      bf16x8 pb[1][1][2], dsb[1][1][2];
      pb[0][0][0] = pack_bf16x8(pe);
      pb[0][0][1] = pack_bf16x8(pe + 8);
      dsb[0][0][0] = pack_bf16x8(ds);
      dsb[0][0][1] = pack_bf16x8(ds + 8);
      pv_tile<D, 1, 1>(sv, dc + kt * 64 * D, rd, pb);   // dV^T += dO^T P
      pv_tile<D, 1, 1>(sk, qc + kt * 64 * D, rd, dsb);  // dK^T += Q^T dS
    }
  }
  if (key_ok) {
    const size_t off = ((size_t)(k_start + key) * p.hkv + kvh) * D;
    store_rows<D>(sk.o[0], p.scale, p.dk, off, p.g_f32, hh);
    store_rows<D>(sv.o[0], 1.f, p.dv, off, p.g_f32, hh);
  }
}

template __global__ void bwd_preprocess_kernel<128>(const BwdParams);
template __global__ void bwd_preprocess_kernel<64>(const BwdParams);
template __global__ void bwd_dq_kernel<128, 4, false>(const BwdParams);
template __global__ void bwd_dq_kernel<128, 4, true>(const BwdParams);
template __global__ void bwd_dq_kernel<64, 4, false>(const BwdParams);
template __global__ void bwd_dq_kernel<64, 4, true>(const BwdParams);
template __global__ void bwd_dkdv_kernel<128, 4, false>(const BwdParams);
template __global__ void bwd_dkdv_kernel<128, 4, true>(const BwdParams);
template __global__ void bwd_dkdv_kernel<64, 4, false>(const BwdParams);
template __global__ void bwd_dkdv_kernel<64, 4, true>(const BwdParams);

constexpr int kBwdWaves = 4;
int bwd_dq_rows() { return kBwdWaves * 32; }
int bwd_dkdv_keys() { return kBwdWaves * 32; }

template <int D, bool CAUSAL>
static hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  const long long pairs = (long long)p.rows_cap * p.hq;
  const int ppb = 256 / (D / 8);
  const int n_kv = p.batch * p.hkv * p.n_kblocks, n_q = p.batch * p.hq * p.n_qtiles;
  // A side with no rows launches nothing: with no queries the dK/dV kernel
  // still runs and writes zeros, with no keys the dQ kernel does.
  if (pairs > 0)
    hipLaunchKernelGGL(bwd_preprocess_kernel<D>, dim3((unsigned)((pairs + ppb - 1) / ppb)),
                       dim3(256), 0, stream, p);
  if (n_kv > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, kBwdWaves, CAUSAL>), dim3(n_kv),
                       dim3(kBwdWaves * 64), 0, stream, p);
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
