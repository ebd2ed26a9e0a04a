// Host program over the LDS tile address helpers of prism_internal.h (the functions the
// attention kernels compile, called here on the host).  It prints, one per line:
//   copy <r0> <lane> <offset of copy 0>              (copy_offset)
//   tr <kb> <db> <lane> <m> <byte offset>           (tr_offset)
//   rm <r> <c> <byte offset>                         (rm_swz)
// and counts where the hoisted forms disagree with the direct ones:
//   xor_row <mismatches>    row_base(t, r) ^ (c << 4)  vs  t + rm_swz(r, c)
//   xor_tr <mismatches>     tr_addr(tr_base(t, lane), m, kb, db)  vs  t + tr_offset(...)
// for 256-byte aligned tiles t.
#include <stdio.h>

#include "../dynamic_block_sparse_stats_amd/csrc/prism_internal.h"

using namespace prism;

int main() {
  for (int r0 = 0; r0 < 64; r0 += 16)
    for (int lane = 0; lane < 64; ++lane) printf("copy %d %d %u\n", r0, lane, copy_offset(r0, lane));
  for (int kb = 0; kb < 64; kb += 16)
    for (int db = 0; db < 128; db += 32)
      for (int lane = 0; lane < 64; ++lane)
        for (int m = 0; m < 2; ++m)
          printf("tr %d %d %d %d %d\n", kb, db, lane, m, tr_offset(kb, db, lane, m));
  for (int r = 0; r < 64; ++r)
    for (int c = 0; c < 16; ++c) printf("rm %d %d %d\n", r, c, rm_swz(r, c));
  const uint32_t tiles[3] = {0u, 49u * 256u, 160u * 1024u - 16384u};
  long bad_row = 0, bad_tr = 0;
  for (uint32_t t : tiles) {
    for (int r = 0; r < 64; ++r)
      for (int c = 0; c < 16; ++c)
        bad_row += (row_base(t, r) ^ (uint32_t)(c << 4)) != t + (uint32_t)rm_swz(r, c);
    for (int lane = 0; lane < 64; ++lane) {
      const TrBase b = tr_base(t, lane);
      for (int kb = 0; kb < 64; kb += 16)
        for (int db = 0; db < 128; db += 32)
          for (int m = 0; m < 2; ++m)
            bad_tr += tr_addr(b, m, kb, db) != t + (uint32_t)tr_offset(kb, db, lane, m);
    }
  }
  printf("xor_row %ld\nxor_tr %ld\n", bad_row, bad_tr);
  return 0;
}
