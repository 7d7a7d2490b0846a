// The attention forward with the score variants the code-reading page lists
// as compile-time switches next to causal masking ("FlashAttention — IO 感知
// 的精确注意力 kernel", section 1 capability table: sliding window, ALiBi,
// softcap): a local window of admissible keys, a per-head linear distance
// bias, and a tanh cap on the scaled scores.  For query i and key j of a
// sequence (delta = Lk - Lq aligns the last query with the last key):
//   x_ij = scale <q_i, k_j>
//   x_ij = cap tanh(x_ij / cap)                      (softcap, cap > 0)
//   x_ij = x_ij - slope_h |i + delta - j|            (ALiBi, slopes given)
//   j admissible: 0 <= j < Lk, and
//     j >= i + delta - left  (left >= 0),  j <= i + delta + right (right >= 0),
//     j <= i + delta         (causal)
//   O_i = softmax over admissible j of x_ij, applied to V;  LSE_i natural log.
//
// Same decomposition as the plain forward (a workgroup per query tile of one
// (sequence, query head), Q fragments in registers, K/V tiles streamed by
// direct loads into the swizzled LDS layout), without its software pipeline:
// each key tile is scored, transformed, masked, folded into the online
// softmax and multiplied into O before the next.  Only the key tiles that
// hold admissible keys of the workgroup's rows are visited, so a window of
// w keys costs about w keys per query.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

// tanh from one exponential: tanh(y) = 1 - 2 / (exp(2y) + 1), which tends to
// +-1 without overflow for large |y|.
__device__ __forceinline__ float tanh_exp(float y) {
  const float e = fast_exp2(y * (2.f * kLog2e));
  return 1.f - 2.f / (e + 1.f);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_ext_kernel(const FwdParams p, const ExtParams x) {
  constexpr int BC = 64;
  constexpr int NKT = BC / 32;
  constexpr int BR = NW * 32;
  constexpr int TILE_BYTES = BC * D * 2;
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE_BYTES];

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
  const int q0 = it * BR;
  if (q0 >= Lq) return;  // packed sequence shorter than this tile (uniform)
  const int delta = Lk - Lq;
  // Admissible keys of query i: [i + delta - left, i + delta + right'] within
  // [0, Lk), right' = min(right, 0) when causal; a negative bound is open.
  const int right = x.causal ? (x.right < 0 ? 0 : min(x.right, 0)) : x.right;
  auto key_lo = [&](int i) { return x.left < 0 ? 0 : max(0, i + delta - x.left); };
  auto key_hi = [&](int i) { return right < 0 ? Lk - 1 : min(Lk - 1, i + delta + right); };
  const int q_last = min(Lq - 1, q0 + BR - 1);
  const int wg_lo = key_lo(q0), wg_hi = key_hi(q_last);
  const int kt0 = wg_lo / BC;
  const int kt1 = wg_hi < wg_lo ? kt0 - 1 : wg_hi / BC;  // last tile (inclusive)
  const int n_kt = kt1 - kt0 + 1;

  const int qw0 = q0 + wave * 32;
  const int qw_last = min(Lq - 1, qw0 + 31);
  const bool wave_active = qw0 < Lq;
  const int w_lo = key_lo(qw0), w_hi = key_hi(qw_last);

  const size_t q_stride = (size_t)p.hq * D;
  const size_t kv_stride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + (size_t)k_start * kv_stride + (size_t)kvh * D;
  const uint16_t* vbase = p.v + (size_t)k_start * kv_stride + (size_t)kvh * D;

  TileDMA<D, BC, NW> dma;
  dma.init(kv_stride, wave, lane);
  LdsRead<D> rd;
  rd.init(lane);
  if (n_kt > 0) {
    dma.issue(kbase, kv_stride, kt0 * BC, Lk - 1, k_lds0, wave, lane);
    dma.issue(vbase, kv_stride, kt0 * BC, Lk - 1, v_lds0, wave, lane);
  }

  WaveState<D, 1> st;
  st.init();
  const int qi = qw0 + m32;
  {
    const uint16_t* qp = p.q + (size_t)(q_start + qi) * q_stride + (size_t)h * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qi < Lq) raw = *reinterpret_cast<const u32x4*>(qp + 16 * s);
      st.qf[0][s] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const int lo_i = key_lo(qi), hi_i = key_hi(qi);  // this lane's admissible keys
  const float slope = x.alibi ? x.alibi[(size_t)b * x.alibi_stride + h] : 0.f;
  const float inv_cap = x.softcap > 0.f ? 1.f / x.softcap : 0.f;

#pragma clang loop unroll(disable)
  for (int j = 0; j < n_kt; ++j) {
    const char* kc = (j & 1) ? k_lds1 : k_lds0;
    const char* vc = (j & 1) ? v_lds1 : v_lds0;
    wait_dma();
    __syncthreads();  // tile j has landed; everyone is done with tile j-1
    if (j + 1 < n_kt) {
      dma.issue(kbase, kv_stride, (kt0 + j + 1) * BC, Lk - 1, (j & 1) ? k_lds0 : k_lds1, wave,
                lane);
      dma.issue(vbase, kv_stride, (kt0 + j + 1) * BC, Lk - 1, (j & 1) ? v_lds0 : v_lds1, wave,
                lane);
    }
    const int k0 = (kt0 + j) * BC;
    // no admissible key of this wave's rows in the tile (uniform)
    if (!wave_active || k0 + BC - 1 < w_lo || k0 > w_hi) continue;
    f32x16 s[NKT][1];
    scores_tile<D, 1, NKT>(s, kc, rd, st.qf);
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kj = k0 + 32 * kt + acc_row(v, hh);
        float y = s[kt][0][v] * x.scale;
        if (inv_cap > 0.f) y = x.softcap * tanh_exp(y * inv_cap);
        y -= slope * fabsf((float)(qi + delta - kj));
        const bool ok = qi < Lq && kj >= lo_i && kj <= hi_i;
        s[kt][0][v] = ok ? y * kLog2e : -INFINITY;
      }
    bf16x8 pb[NKT][1][2];
    softmax_update<D, 1, NKT>(st, s, pb, 1.f);
    pv_tile<D, 1, NKT>(st, vc, rd, pb);
  }

  // ---- epilogue: O / l, LSE = ln 2 * (r + log2 l) ----
  const float lt = halfwave_sum(st.l[0]);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (st.mc[0] + __log2f(lt)) * kLn2 : -INFINITY;
  if (qi < Lq) {
    const size_t orow = (size_t)(q_start + qi) * p.hq + h;
    if (p.o_f32) {
      float* op = reinterpret_cast<float*>(p.o) + orow * D + 4 * hh;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w = {st.o[0][dt][4 * g] * inv, st.o[0][dt][4 * g + 1] * inv,
                     st.o[0][dt][4 * g + 2] * inv, st.o[0][dt][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(op + dt * 32 + 8 * g) = w;
        }
    } else {
      uint16_t* op = reinterpret_cast<uint16_t*>(p.o) + orow * D + 4 * hh;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w = {pack_bf16x2(st.o[0][dt][4 * g] * inv, st.o[0][dt][4 * g + 1] * inv),
                     pack_bf16x2(st.o[0][dt][4 * g + 2] * inv, st.o[0][dt][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(op + dt * 32 + 8 * g) = w;
        }
    }
    if (hh == 0) p.lse[orow] = lse;
  }
}

template __global__ void fwd_ext_kernel<128, 4>(const FwdParams, const ExtParams);
template __global__ void fwd_ext_kernel<64, 4>(const FwdParams, const ExtParams);

int fwd_ext_rows() { return 4 * 32; }

hipError_t launch_fwd_ext(const FwdParams& p, const ExtParams& x, int head_dim,
                          hipStream_t stream) {
  if (head_dim == 128)
    hipLaunchKernelGGL((fwd_ext_kernel<128, 4>), dim3(p.total), dim3(256), 0, stream, p, x);
  else
    hipLaunchKernelGGL((fwd_ext_kernel<64, 4>), dim3(p.total), dim3(256), 0, stream, p, x);
  return hipGetLastError();
}

}  // namespace fa
