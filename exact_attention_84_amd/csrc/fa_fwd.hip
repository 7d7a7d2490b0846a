// Fused attention forward (prefill): fixed-length batches and packed
// variable-length sequences, causal or not, MHA or GQA.
//
// Work decomposition: one workgroup per (sequence, query head, tile of BR
// query rows); the Q tile stays in registers while K/V tiles of BC keys
// stream through LDS ("FlashAttention — IO 感知的精确注意力 kernel", section
// 2.3 step 4: one Q tile per thread block, K/V tiles streamed through on-chip
// memory, launched over (Q blocks, batch, head)).  Causal tiles stop at the
// diagonal, so a causal forward does about half the work ("推理优化 |
// FlashAttention 1-4 详解", section FlashAttention 2 的工程优化, causal
// lower-triangle skipping).  Masks are applied only on tiles that cross the
// diagonal or the end of the keys.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

// Two waves per SIMD (256 registers each) when a wave owns 32 query rows, so
// that one wave's MFMAs overlap the other's softmax arithmetic.
template <int D, int NW, int NT, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 2 : 1)))
void fwd_kernel(const FwdParams p) {
  constexpr int BC = 64;
  constexpr int BR = NW * 32 * NT;
  constexpr int TILE_BYTES = BC * D * 2;
  // Two stages of K and V: the next tile streams in while this one is used.
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int m32 = lane & 31, hh = lane >> 5;

  // ---- work item: (sequence b, kv head, query head in group, query tile) ----
  const int item = xcd_remap(blockIdx.x, p.total);
  const int qt_r = item % p.n_qtiles;
  int rest = item / p.n_qtiles;
  const int hg = rest % p.group;
  rest /= p.group;
  const int kvh = rest % p.hkv;
  const int b = rest / p.hkv;
  const int h = kvh * p.group + hg;
  // Causal tiles are heaviest at the end of the sequence: start those first.
  const int qt = CAUSAL ? p.n_qtiles - 1 - qt_r : qt_r;

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
  const int q0 = qt * BR;
  if (q0 >= Lq) return;  // packed sequence shorter than this tile (uniform)

  const int delta = Lk - Lq;  // bottom-right causal offset
  int n_kt = (Lk + BC - 1) / BC;
  if (CAUSAL) {
    const int last_key = min(Lk - 1, q0 + BR - 1 + delta);
    n_kt = last_key < 0 ? 0 : min(n_kt, last_key / BC + 1);
  }
  const int qw0 = q0 + wave * 32 * NT;
  const bool wave_active = qw0 < Lq;
  const int wave_last_key = CAUSAL ? min(Lk - 1, qw0 + 32 * NT - 1 + delta) : Lk - 1;

  const size_t q_stride = (size_t)p.hq * D;
  const size_t kv_stride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + (size_t)k_start * kv_stride + (size_t)kvh * D;
  const uint16_t* vbase = p.v + (size_t)k_start * kv_stride + (size_t)kvh * D;

  TileDMA<D, BC, NW> dma;
  dma.init(kv_stride, wave, lane);
  if (n_kt > 0) {
    dma.issue(kbase, kv_stride, 0, Lk - 1, k_lds0, wave, lane);
    dma.issue(vbase, kv_stride, 0, Lk - 1, v_lds0, wave, lane);
  }

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

  for (int j = 0; j < n_kt; ++j) {
    const int k0 = j * BC;
    wait_dma();       // this wave's share of tile j has landed in LDS
    __syncthreads();  // everyone's share has; everyone is done with tile j-1
    const char* k_cur = (j & 1) ? k_lds1 : k_lds0;
    const char* v_cur = (j & 1) ? v_lds1 : v_lds0;
    if (j + 1 < n_kt) {
      dma.issue(kbase, kv_stride, k0 + BC, Lk - 1, (j & 1) ? k_lds0 : k_lds1, wave, lane);
      dma.issue(vbase, kv_stride, k0 + BC, Lk - 1, (j & 1) ? v_lds0 : v_lds1, wave, lane);
    }

    if (wave_active && k0 <= wave_last_key) {
      f32x16 s[BC / 32][NT];
      scores_tile<D, NT, BC / 32>(s, k_cur, 0, st.qf, m32, hh);

      const bool edge = (k0 + BC > Lk) || (CAUSAL && k0 + BC - 1 > qw0 + delta);
      if (edge) {
#pragma unroll
        for (int kt = 0; kt < BC / 32; ++kt)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int qi = qw0 + t * 32 + m32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int key = k0 + kt * 32 + acc_row(v, hh);
              const bool ok = key < Lk && (!CAUSAL || key <= qi + delta);
              if (!ok) s[kt][t][v] = -INFINITY;
            }
          }
      }

      bf16x8 pb[BC / 32][NT][2];
      softmax_update<D, NT, BC / 32>(st, s, pb, p.c);
      pv_tile<D, NT, BC / 32>(st, v_cur, 0, pb, lane);
    }
  }

  // ---- epilogue: O / l, LSE = ln 2 * (m c + log2 l) ----
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lt = halfwave_sum(st.l[t]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (st.mc[t] + __log2f(lt)) * kLn2 : -INFINITY;
    const int qi = qw0 + t * 32 + m32;
    if (qi < Lq) {
      const size_t orow = (size_t)(q_start + qi) * p.hq + h;
      if (p.o_f32) {
        float* op = reinterpret_cast<float*>(p.o) + orow * D + 4 * hh;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 w = {st.o[t][dt][4 * g] * inv, st.o[t][dt][4 * g + 1] * inv,
                       st.o[t][dt][4 * g + 2] * inv, st.o[t][dt][4 * g + 3] * inv};
            *reinterpret_cast<f32x4*>(op + dt * 32 + 8 * g) = w;
          }
      } else {
        uint16_t* op = reinterpret_cast<uint16_t*>(p.o) + orow * D + 4 * hh;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u32x2 w = {pack_bf16x2(st.o[t][dt][4 * g] * inv, st.o[t][dt][4 * g + 1] * inv),
                       pack_bf16x2(st.o[t][dt][4 * g + 2] * inv, st.o[t][dt][4 * g + 3] * inv)};
            *reinterpret_cast<u32x2*>(op + dt * 32 + 8 * g) = w;
          }
      }
      if (hh == 0) p.lse[orow] = lse;
    }
  }
}

// Explicit instantiations: every kernel the dispatcher can launch is emitted
// on both the device and the host side.
template __global__ void fwd_kernel<128, kFwdWaves, kFwdNT, false>(const FwdParams);
template __global__ void fwd_kernel<128, kFwdWaves, kFwdNT, true>(const FwdParams);
template __global__ void fwd_kernel<64, kFwdWaves, kFwdNT, false>(const FwdParams);
template __global__ void fwd_kernel<64, kFwdWaves, kFwdNT, true>(const FwdParams);

template <int D, int NW, int NT, bool CAUSAL>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_kernel<D, NW, NT, CAUSAL>), dim3(p.total), dim3(NW * 64), 0, stream,
                     p);
  return hipGetLastError();
}

int fwd_block_rows(int head_dim) {
  (void)head_dim;
  return kFwdWaves * 32 * kFwdNT;
}

hipError_t launch_fwd(const FwdParams& p, int head_dim, bool causal, hipStream_t stream) {
  if (head_dim == 128)
    return causal ? launch_one<128, kFwdWaves, kFwdNT, true>(p, stream)
                  : launch_one<128, kFwdWaves, kFwdNT, false>(p, stream);
  return causal ? launch_one<64, kFwdWaves, kFwdNT, true>(p, stream)
                : launch_one<64, kFwdWaves, kFwdNT, false>(p, stream);
}

}  // namespace fa
