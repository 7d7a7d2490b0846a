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

// ---------------------------------------------------------------------------
// FP8 (E4M3) tiles, head dim 128: row r (one key) holds 128 one-byte values,
// 8 chunks of 16 bytes, two rows per 256-byte bank cycle.
//
// Both products use v_mfma_scale_f32_32x32x64_f8f6f4, whose A and B operands
// give every lane 32 bytes (byte s = slot s).  The two operands pair their
// slots identically, so any assignment of the contraction index to (half-wave
// hh, slot s) that both operands follow gives the product:
//   * S^T = K Q^T: head-dim index 64 st + 32 hh + s for k-step st, i.e. 32
//     consecutive bytes of the key row (A) and of the query row (B);
//   * O^T = V^T P^T: key pv8_key(hh, s) of the 64-key tile, the key that
//     element s = 16 kt + v of the lane's S^T accumulators holds, so P goes
//     from the accumulators into the B operand in order.
// ---------------------------------------------------------------------------
FA_HD constexpr int pv8_key(int hh, int s) {
  return ((s & 15) & 3) + 8 * ((s & 15) >> 2) + 4 * hh + 32 * (s >> 4);
}

// K tile swizzle: the 16 rows one 16-byte operand read serves per clock
// (rows r0..r0+15, one logical chunk) land on 16 distinct 16-byte bank groups.
FA_HD constexpr int k8_swizzle(int r) { return (r >> 1) & 7; }
// V tile swizzle: the 32 lanes one transposing read serves per clock (8 key
// rows {0..3, 8..11} + 4 hh + 16 q, two logical chunks, two 8-byte halves)
// land on 16 distinct bank groups, two halves each.
FA_HD constexpr int v8_swizzle(int r) { return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2); }

FA_HD constexpr int k8_offset(int row, int chunk) {
  return row * 128 + ((chunk ^ k8_swizzle(row)) << 4);
}
FA_HD constexpr int v8_offset(int row, int chunk) {
  return row * 128 + ((chunk ^ v8_swizzle(row)) << 4);
}

// DMA of an FP8 tile: wave instruction i writes bytes [1024 i, +1024), lane l
// the 16 bytes of row 8 i + l / 8 at physical chunk l % 8, which hold logical
// chunk dma8_chunk(...) of that row.
FA_HD constexpr int dma8_row(int inst, int lane) { return 8 * inst + lane / 8; }
FA_HD constexpr int dma8_chunk(int inst, int lane, bool v_tile) {
  return (lane % 8) ^ (v_tile ? v8_swizzle(dma8_row(inst, lane)) : k8_swizzle(dma8_row(inst, lane)));
}

// A operand of S^T = K Q^T, k-step st, 16-byte half u of the lane's 32 bytes:
// key row lane % 32 (+32 kt adds 4096 bytes: same swizzle), logical chunk
// 4 st + 2 hh + u.
FA_HD constexpr int k8_read_offset(int lane, int st, int u) {
  return k8_offset(lane & 31, 4 * st + 2 * (lane >> 5) + u);
}

// A operand of O^T = V^T P^T for head-dim rows 32 dt.. with four transposing
// reads (ds_read_b64_tr_b8), read q giving slots 8 q .. 8 q + 7.  Within each
// group of 16 lanes that read hands result lane i, byte j, the byte i % 8 of
// the 8 bytes source lane 2 j + (i / 8) % 2 addressed.  So source lane s of
// group g (j = (s % 16) / 2, c = s % 2, hh = g / 2) addresses key row
// pv8_key(hh, 8 q + j) and head-dim columns 32 dt + 16 (g % 2) + 8 c .. +7:
// logical chunk 2 dt + g % 2, half c.  Read q adds 16 q rows (2048 q bytes;
// the swizzle does not see row bits 4 and 5).
FA_HD constexpr int v8_read_offset(int lane, int dt) {
  const int g = (lane & 63) >> 4, j = (lane & 15) >> 1, c = lane & 1, hh = g >> 1;
  return v8_offset(pv8_key(hh, j), 2 * dt + (g & 1)) + 8 * c;
}

}  // namespace fa
