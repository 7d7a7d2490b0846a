// Integer layout of the K and V tiles in LDS and of the MFMA operand reads
// (host and device code, no intrinsics), so that host-side tests can check
// the exact offsets the kernels use.
//
// Tiles are row-major: row r (one key) holds D bf16 values, 2 D bytes, split
// into D / 8 chunks of 16 bytes.  The chunk index is XOR-swizzled by sw(r).
// gfx950's LDS has 64 banks of 4 bytes: a 16-byte read serves 16 lanes per
// clock, an 8-byte read 32 lanes.  sw puts on distinct banks (a) the 16
// consecutive rows of one K operand read, all at the same logical chunk, and
// (b) the 4 rows x 4 chunks of the 32 lanes of one transposing V read.
#pragma once

#if defined(__HIPCC__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

namespace fa {

template <int D>
FA_HD constexpr int kv_swizzle(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3))          // 16 chunks per row
                  : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));  // 8 chunks per row
}

// Byte offset of logical chunk `chunk` of tile row `row`.
template <int D>
FA_HD constexpr int kv_offset(int row, int chunk) {
  return row * (2 * D) + ((chunk ^ kv_swizzle<D>(row)) << 4);
}

// The tile is filled by wave instructions that each write 64 x 16 consecutive
// bytes: lane `lane` of instruction i writes bytes [1024 i + 16 lane, +16),
// i.e. tile row i * (64 / (D/8)) + lane / (D/8), physical chunk lane % (D/8),
// which holds logical chunk dma_chunk(...) of that row.
template <int D>
FA_HD constexpr int dma_row(int inst, int lane) {
  return inst * (64 / (D / 8)) + lane / (D / 8);
}
template <int D>
FA_HD constexpr int dma_chunk(int inst, int lane) {
  return (lane % (D / 8)) ^ kv_swizzle<D>(dma_row<D>(inst, lane));
}

// A operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16): lane l reads the 8
// values of key row (l % 32) at head-dim 16 st + 8 (l / 32).  Rows kt*32 + r
// share the swizzle of r, so sub-tile kt adds 64 D bytes.
template <int D>
FA_HD constexpr int k_read_offset(int lane, int st) {
  return kv_offset<D>(lane & 31, 2 * st + (lane >> 5));
}

// One of the two transposing reads (ds_read_b64_tr_b16) of the A operand of
// O^T = V^T P^T for head-dim rows dt*32..: source lane k of 16-lane group g
// addresses key row 4 (l / 32) + (k >> 2) (+8 for the second read, sec = 1)
// and head-dim columns dt*32 + 16 (g & 1) + 4 (k & 3) .. +3, i.e. half
// (k & 1) of chunk dt*4 + 2 (g & 1) + ((k & 3) >> 1).  The 16-key step
// (kt, u) adds (32 kt + 16 u) rows.
template <int D>
FA_HD constexpr int v_read_offset(int lane, int dt, int sec) {
  const int k = lane & 15, g = lane >> 4, hh = lane >> 5;
  return kv_offset<D>(4 * hh + (k >> 2) + 8 * sec, dt * 4 + 2 * (g & 1) + ((k & 3) >> 1)) +
         8 * (k & 1);
}

}  // namespace fa
