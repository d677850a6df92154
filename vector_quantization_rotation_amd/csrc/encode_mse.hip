// Algorithm 1 instantiations of the fused encode (encode.cuh).
#include "encode.cuh"

namespace tq {

template <int XT, int D>
static void mse_bits(int bm, const EncArgs &ea, hipStream_t st) {
  switch (bm) {
    case 1: launch_encode<XT, D, false, 1>(ea, st); break;
    case 2: launch_encode<XT, D, false, 2>(ea, st); break;
    case 3: launch_encode<XT, D, false, 3>(ea, st); break;
    default: launch_encode<XT, D, false, 4>(ea, st); break;
  }
}

void launch_encode_mse(int xt, int d, int bm, const EncArgs &ea, hipStream_t st) {
  if (d == 128) {
    if (xt == TQ_F32) mse_bits<TQ_F32, 128>(bm, ea, st);
    else if (xt == TQ_BF16) mse_bits<TQ_BF16, 128>(bm, ea, st);
    else mse_bits<TQ_F16, 128>(bm, ea, st);
  } else {
    if (xt == TQ_F32) mse_bits<TQ_F32, 64>(bm, ea, st);
    else if (xt == TQ_BF16) mse_bits<TQ_BF16, 64>(bm, ea, st);
    else mse_bits<TQ_F16, 64>(bm, ea, st);
  }
}

}  // namespace tq
