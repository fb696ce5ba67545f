// The decode-attention kernels for caches quantized in groups of 16 tokens
// (keys) and 16 channels (values), MiniKV Sec. 5.1's group size: the MFMA
// kernel of decode_kernel.h instantiated with GS = 16, in a translation unit of
// its own so that the two group sizes compile in parallel.
#include "decode_kernel.h"

namespace kvc {

const void* kernel_for_g16(int dt, int bits, int KS, int nwv, int hbs) {
  return kernel_for_gs<16>(dt, bits, KS, nwv, hbs);
}

}  // namespace kvc
