// Host build of the library's double-double GeLU (zk_gelu_exact.h, the
// forward kernels' path for arguments their table cannot round with
// certainty), for tests/test_host.py: reads binary32 bit patterns (hex, one
// a line) on stdin and writes the bit pattern of gelu32_exact for each.
#include <cstdio>
#include <cstring>

#include "zk_gelu_exact.h"

int main() {
  unsigned u;
  while (std::scanf("%x", &u) == 1) {
    float h;
    std::memcpy(&h, &u, 4);
    const float y = zk::gelu32_exact(h);
    unsigned v;
    std::memcpy(&v, &y, 4);
    std::printf("%08x\n", v);
  }
  return 0;
}
