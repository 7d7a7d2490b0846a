// Host program for tests/test_lds_layout.py: prints, for each head dim, the
// LDS offsets the attention kernels use (tile fill by direct loads, K operand
// reads, transposing V operand reads), computed by the kernels' own layout
// header.
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

int main() {
  dump<128>();
  dump<64>();
  return 0;
}
