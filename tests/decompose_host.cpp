// Host harness of the work decomposition (test infrastructure, built by tests/test_decompose.py):
// prints, for every hardware workgroup id 0 .. nqb*Hq*B-1 of one grid, the (query block, head,
// sequence) the kernels' decompose() assigns to it, as three int32 values per workgroup.
//   usage: decompose_host nqb Hq Hkv B causal
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "decompose.h"

int main(int argc, char** argv) {
  if (argc != 6) {
    fprintf(stderr, "usage: %s nqb Hq Hkv B causal\n", argv[0]);
    return 2;
  }
  const int nqb = atoi(argv[1]), Hq = atoi(argv[2]), Hkv = atoi(argv[3]), B = atoi(argv[4]);
  const bool causal = atoi(argv[5]) != 0;
  const long long total = (long long)nqb * Hq * B;
  for (long long wg = 0; wg < total; ++wg) {
    int32_t out[3];
    int qb, h, b;
    if (causal) attn::decompose<true>((int)wg, nqb, Hq, Hkv, B, qb, h, b);
    else attn::decompose<false>((int)wg, nqb, Hq, Hkv, B, qb, h, b);
    out[0] = qb;
    out[1] = h;
    out[2] = b;
    fwrite(out, sizeof(out), 1, stdout);
  }
  return 0;
}
