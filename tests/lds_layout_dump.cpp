// Host program for tests/test_lds_layout.py: prints, for each head dim, the
// LDS offsets the attention kernels use (tile fill by direct loads, K operand
// reads, transposing V operand reads), computed by the kernels' own layout
// header; with an argument, the same for the FP8 tiles.
#include <cstdio>

#include "fa_layout.hpp"

template <int D>
void dump() {
  std::printf("D %d\n", D);
  for (int inst = 0; inst < 64 / (64 / (D / 8)); ++inst)
    for (int lane = 0; lane < 64; ++lane)
      std::printf("dma %d %d %d %d\n", inst, lane, fa::dma_row<D>(inst, lane),
                  fa::dma_chunk<D>(inst, lane));
  for (int st = 0; st < D / 16; ++st)
    for (int lane = 0; lane < 64; ++lane)
      std::printf("k %d %d %d\n", st, lane, fa::k_read_offset<D>(lane, st));
  for (int dt = 0; dt < D / 32; ++dt)
    for (int sec = 0; sec < 2; ++sec)
      for (int lane = 0; lane < 64; ++lane)
        std::printf("v %d %d %d %d\n", dt, sec, lane, fa::v_read_offset<D>(lane, dt, sec));
}

// FP8 tiles (head dim 128): DMA fill of K (kind 0) and V (kind 1) tiles, K
// operand reads, transposing V operand reads, and the key of each P slot.
void dump_fp8() {
  for (int kind = 0; kind < 2; ++kind)
    for (int inst = 0; inst < 8; ++inst)
      for (int lane = 0; lane < 64; ++lane)
        std::printf("dma %d %d %d %d %d\n", kind, inst, lane, fa::dma8_row(inst, lane),
                    fa::dma8_chunk(inst, lane, kind == 1));
  for (int st = 0; st < 2; ++st)
    for (int u = 0; u < 2; ++u)
      for (int lane = 0; lane < 64; ++lane)
        std::printf("k %d %d %d %d\n", st, u, lane, fa::k8_read_offset(lane, st, u));
  for (int dt = 0; dt < 4; ++dt)
    for (int lane = 0; lane < 64; ++lane)
      std::printf("v %d %d %d\n", dt, lane, fa::v8_read_offset(lane, dt));
  for (int hh = 0; hh < 2; ++hh)
    for (int s = 0; s < 32; ++s) std::printf("p %d %d %d\n", hh, s, fa::pv8_key(hh, s));
}

int main(int argc, char** argv) {
  if (argc > 1) {
    dump_fp8();
    return 0;
  }
  dump<128>();
  dump<64>();
  return 0;
}
