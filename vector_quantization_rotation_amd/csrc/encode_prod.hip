// Algorithm 2 instantiations of the fused encode (encode.cuh): the Algorithm 1
// part runs at b - 1 bits.
#include "encode.cuh"

namespace tq {

template <int XT, int D>
static void prod_bits(int bm, const EncArgs &ea, hipStream_t st) {
  switch (bm) {
    case 1: launch_encode<XT, D, true, 1>(ea, st); break;
    case 2: launch_encode<XT, D, true, 2>(ea, st); break;
    default: launch_encode<XT, D, true, 3>(ea, st); break;
  }
}

void launch_encode_prod(int xt, int d, int bm, const EncArgs &ea, hipStream_t st) {
  if (d == 128) {
    if (xt == TQ_F32) prod_bits<TQ_F32, 128>(bm, ea, st);
    else if (xt == TQ_BF16) prod_bits<TQ_BF16, 128>(bm, ea, st);
    else prod_bits<TQ_F16, 128>(bm, ea, st);
  } else {
    if (xt == TQ_F32) prod_bits<TQ_F32, 64>(bm, ea, st);
    else if (xt == TQ_BF16) prod_bits<TQ_BF16, 64>(bm, ea, st);
    else prod_bits<TQ_F16, 64>(bm, ea, st);
  }
}

}  // namespace tq
