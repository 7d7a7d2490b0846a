// Split-KV decode (one query per sequence against a KV cache) and the
// LSE-weighted combine of partial results.
//
// The G = Hq / Hkv query heads that share a key/value head are folded into the
// query-row dimension ("FlashAttention — IO 感知的精确注意力 kernel", section
// 4: at decode time with grouped heads, the group dimension is reshaped into
// the sequence dimension), so one workgroup serves a whole group from a single
// read of its keys.  The cache of each sequence is cut into chunks processed
// by separate workgroups (split-KV for a short query against long keys, same
// page, section 2.3 step 3); each chunk writes its normalised partial output
// and logsumexp, and a second kernel merges them by LSE weight (the block
// merge of the PKU lecture notes "FlashAttention", section 6: only the
// running max, sum and output of each part are kept).
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

template <int D>
__global__ __launch_bounds__(kDecodeWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_kernel(const DecodeParams p) {
  constexpr int BC = kDecodeTile;
  constexpr int T = kDecodeWaves * 64;
  static_assert(BC == 32 * kDecodeWaves, "one 32-key sub-tile per wave");
  constexpr int CPR = D / 8;             // 16-byte chunks per key row
  constexpr int NCH = BC * CPR / T;      // chunks per thread, per tensor
  constexpr int TILE = BC * D * 2;       // bytes of one K or V tile
  constexpr int MERGE = kDecodeWaves * kDecodeMaxGroup * (D + 2) * 4;
  constexpr int SMEM = 2 * TILE > MERGE ? 2 * TILE : MERGE;
  static_assert(BC * CPR % T == 0, "tile chunks must split evenly over the threads");
  // K and V tiles row-major with the XOR-swizzled chunk layout of fa_layout.hpp
  // (conflict-free operand reads on 64 banks); the area is reused for the
  // cross-wave merge at the end.
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  char* k_lds = smem;
  char* v_lds = smem + TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int m32 = lane & 31, hh = lane >> 5;

  int item = blockIdx.x;
  const int split = item % p.n_splits;
  item /= p.n_splits;
  const int kvh = item % p.hkv;
  const int b = item / p.hkv;
  const int G = p.group;
  // Lengths are clamped to the cache so that a bad length cannot read past it.
  const int Lk = min(max(p.cache_seqlens[b] + p.len_add, 0), p.cache_len);
  const int kbeg = split * p.chunk;
  const int kend = min(Lk, kbeg + p.chunk);
  const size_t row0 = (size_t)b * p.hq + (size_t)kvh * G;  // output row of head kvh*G
  if (kbeg >= kend) {
    if (tid < G) p.lse_part[(row0 + tid) * p.n_splits + split] = -INFINITY;
    return;
  }

  const size_t kv_stride = (size_t)p.hkv * D;
  // First row of the 128-key tile at k0 (one tile never straddles a page: the
  // page size is a multiple of the tile and tiles start at multiples of it).
  // Block ids are clamped to the pool so that a bad table cannot read past it.
  auto tile_row = [&](int k0) -> size_t {
    if (p.block_table) {
      int blk = p.block_table[(size_t)b * p.max_blocks + k0 / p.page_size];
      blk = min(max(blk, 0), p.num_blocks - 1);
      return (size_t)blk * p.page_size + k0 % p.page_size;
    }
    return (size_t)b * p.cache_len + k0;
  };

  WaveState<D, 1> st;
  st.init();
  {
    const uint16_t* qp = p.q + (row0 + m32) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (m32 < G) raw = *reinterpret_cast<const u32x4*>(qp + 16 * s);
      st.qf[0][s] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  LdsRead<D> rd;
  rd.init(lane);

  // Next tile staged in registers while this one is used: thread tid moves
  // chunks tid + i*T (row c / CPR, chunk c % CPR) of K and of V.  Keys past
  // the end are zero (their scores are masked; zero V rows add nothing).
  u32x4 kr[NCH], vr[NCH];
  auto load = [&](int k0) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const size_t base = tile_row(k0) * kv_stride + (size_t)kvh * D;
    const uint16_t* kt = p.k + base;
    const uint16_t* vt = p.v + base;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * T;
      const int key = k0 + c / CPR;
      const size_t off = (size_t)(c / CPR) * kv_stride + (c % CPR) * 8;
      kr[i] = key < kend ? *reinterpret_cast<const u32x4*>(kt + off) : zero;
      vr[i] = key < kend ? *reinterpret_cast<const u32x4*>(vt + off) : zero;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * T;
      const int o = kv_offset<D>(c / CPR, c % CPR);
      *reinterpret_cast<u32x4*>(k_lds + o) = kr[i];
      *reinterpret_cast<u32x4*>(v_lds + o) = vr[i];
    }
  };

  load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += BC) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + BC < kend) load(k0 + BC);

    const int ksub = k0 + wave * 32;  // this wave's 32 keys of the tile
    if (ksub < kend) {
      f32x16 s[1][1];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        s[0][0] = mfma_32x32x16(rd.k(k_lds, wave, ks), st.qf[0][ks],
                                ks == 0 ? f32x16{} : s[0][0]);
      if (ksub + 32 > kend) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (ksub + acc_row(v, hh) >= kend) s[0][0][v] = -INFINITY;
      }
      bf16x8 pb[1][1][2];
      softmax_update<D, 1, 1>(st, s, pb, p.c);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          st.o[0][dt] = mfma_32x32x16(rd.v(v_lds, wave, u, dt), pb[0][0][u], st.o[0][dt]);
    }
  }

  // ---- merge the four waves' key subsets, then write this chunk's partial ----
  __syncthreads();  // the K/V staging area becomes the merge buffer
  float* red_o = reinterpret_cast<float*>(smem);         // [waves][G][D]
  float* red_m = red_o + kDecodeWaves * G * D;           // [waves][G]
  float* red_l = red_m + kDecodeWaves * G;               // [waves][G]
  const float lt = halfwave_sum(st.l[0]);
  if (m32 < G) {
    float* ro = red_o + (wave * G + m32) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) ro[dt * 32 + acc_row(v, hh)] = st.o[0][dt][v];
    if (hh == 0) {
      red_m[wave * G + m32] = st.mc[0];
      red_l[wave * G + m32] = lt;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += T) {
    const int n = idx / D, d = idx % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) mx = fmaxf(mx, red_m[w * G + n]);
    const float msub = mx == -INFINITY ? 0.f : mx;
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float f = fast_exp2(red_m[w * G + n] - msub);
      lsum += f * red_l[w * G + n];
      acc += f * red_o[(w * G + n) * D + d];
    }
    const size_t row = row0 + n;
    p.o_part[(row * p.n_splits + split) * D + d] = lsum > 0.f ? acc / lsum : 0.f;
    if (d == 0)
      p.lse_part[row * p.n_splits + split] =
          lsum > 0.f ? (mx + __log2f(lsum)) * kLn2 : -INFINITY;
  }
}

// In-place append of each sequence's new token, with rotary embedding: one
// thread per element of a query row (rotated into q_rot) or a new key row
// (rotated, then written to cache row t = cache_seqlens[b] with the new value
// row).  Pair i of the first rdim components turns by the angle of table row
// t: (a, b) -> (a cos - b sin, b cos + a sin), with pairs (i, i + rdim/2) or
// (2i, 2i + 1) when interleaved; the products and the difference are rounded
// separately (no fused multiply-add), then the result is rounded to bf16.
// Positions outside the table are not rotated and rows outside the cache are
// not written (preconditions of the call; never an out-of-bounds access).
template <int D>
__global__ __launch_bounds__(256) void append_kernel(const AppendParams a) {
  constexpr int RPB = 256 / D;
  const int r = blockIdx.x * RPB + threadIdx.x / D;
  const int e = threadIdx.x % D;
  const int per = a.hq + a.hkv;
  if (r >= a.batch * per) return;
  const int b = r / per, h = r % per;
  const bool is_q = h < a.hq;
  if (is_q && !a.q_rot) return;
  if (!is_q && !a.k_new) return;
  const int t = a.cache_seqlens[b];
  const uint16_t* src = is_q ? a.q + ((size_t)b * a.hq + h) * D
                             : a.k_new + ((size_t)b * a.hkv + (h - a.hq)) * D;
  auto f32 = [](uint16_t u) { return __builtin_bit_cast(float, (uint32_t)u << 16); };
  float out = f32(src[e]);
  if (a.cos && t >= 0 && t < a.max_pos && e < a.rdim) {
    const int half = a.rdim / 2;
    int i, ia, ib;
    if (a.interleaved) {
      i = e >> 1;
      ia = 2 * i;
      ib = 2 * i + 1;
    } else {
      i = e < half ? e : e - half;
      ia = i;
      ib = i + half;
    }
    const float x = f32(src[ia]), y = f32(src[ib]);
    const float cs = a.cos[(size_t)t * half + i], sn = a.sin[(size_t)t * half + i];
    {
#pragma clang fp contract(off)
      const float p1 = (e == ia ? x : y) * cs;
      const float p2 = (e == ia ? y : x) * sn;
      out = e == ia ? p1 - p2 : p1 + p2;
    }
  }
  const uint16_t bits = __builtin_bit_cast(uint16_t, (__bf16)out);
  if (is_q) {
    a.q_rot[((size_t)b * a.hq + h) * D + e] = bits;
    return;
  }
  if (t < 0 || t >= a.cache_len) return;
  size_t row;
  if (a.block_table) {
    int blk = a.block_table[(size_t)b * a.max_blocks + t / a.page_size];
    blk = min(max(blk, 0), a.num_blocks - 1);
    row = (size_t)blk * a.page_size + t % a.page_size;
  } else {
    row = (size_t)b * a.cache_len + t;
  }
  const int kvh = h - a.hq;
  const size_t dst = (row * a.hkv + kvh) * D + e;
  a.k_cache[dst] = bits;
  a.v_cache[dst] = a.v_new[((size_t)b * a.hkv + kvh) * D + e];
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// One wave per output row: M = max_s lse_s, lse = M + ln sum_s exp(lse_s - M),
// o = sum_s exp(lse_s - lse) o_s over the non-empty splits.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part, int rows,
                                                      int n_splits, void* o, float* lse,
                                                      int o_f32) {
  constexpr int PER = D / 64;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* lp = lse_part + (size_t)row * n_splits;
  float mx = -INFINITY;
  for (int s = lane; s < n_splits; s += 64) mx = fmaxf(mx, lp[s]);
  mx = wave_max(mx);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float out_lse = -INFINITY;
  if (mx != -INFINITY) {
    float sum = 0.f;
    for (int s = lane; s < n_splits; s += 64) {
      const float x = lp[s];
      sum += (x == -INFINITY) ? 0.f : expf(x - mx);
    }
    sum = wave_sum(sum);
    out_lse = mx + logf(sum);
    const float* op = o_part + (size_t)row * n_splits * D + lane * PER;
    // Four splits at a time, their loads issued together (the loop is bound
    // by load latency, not bandwidth).  An empty split (LSE = -inf) never
    // wrote its partial O, so its values are read but not used.
    constexpr int U = 4;
    int s = 0;
    for (; s + U <= n_splits; s += U) {
      float x[U], v[U][PER];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        x[u] = lp[s + u];
#pragma unroll
        for (int e = 0; e < PER; ++e) v[u][e] = op[(size_t)(s + u) * D + e];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (x[u] == -INFINITY) continue;
        const float w = expf(x[u] - out_lse);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += w * v[u][e];
      }
    }
    for (; s < n_splits; ++s) {
      const float x = lp[s];
      if (x == -INFINITY) continue;
      const float w = expf(x - out_lse);
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += w * op[(size_t)s * D + e];
    }
  }
  if (o_f32) {
    float* dst = reinterpret_cast<float*>(o) + (size_t)row * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e] = acc[e];
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(o) + (size_t)row * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; e += 2) *reinterpret_cast<uint32_t*>(dst + e) = pack_bf16x2(acc[e], acc[e + 1]);
  }
  if (lane == 0) lse[row] = out_lse;
}

template __global__ void decode_kernel<128>(const DecodeParams);
template __global__ void decode_kernel<64>(const DecodeParams);
template __global__ void combine_kernel<128>(const float*, const float*, int, int, void*, float*,
                                             int);
template __global__ void combine_kernel<64>(const float*, const float*, int, int, void*, float*,
                                            int);

hipError_t launch_append(const AppendParams& a, int head_dim, hipStream_t stream) {
  const long long rows = (long long)a.batch * (a.hq + a.hkv);
  const int rpb = 256 / head_dim;
  const unsigned blocks = (unsigned)((rows + rpb - 1) / rpb);
  if (blocks == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(append_kernel<128>, dim3(blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<64>, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 128)
    hipLaunchKernelGGL(decode_kernel<128>, dim3(p.total), dim3(kDecodeWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_kernel<64>, dim3(p.total), dim3(kDecodeWaves * 64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(const float* o_part, const float* lse_part, int rows, int n_splits,
                          int head_dim, void* o, float* lse, int o_f32, hipStream_t stream) {
  const dim3 grid((rows + 3) / 4);
  if (head_dim == 128)
    hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(256), 0, stream, o_part, lse_part, rows,
                       n_splits, o, lse, o_f32);
  else
    hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(256), 0, stream, o_part, lse_part, rows,
                       n_splits, o, lse, o_f32);
  return hipGetLastError();
}

}  // namespace fa
