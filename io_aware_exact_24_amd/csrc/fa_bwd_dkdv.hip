// dK/dV launcher of the backward pass (kernel in fa_bwd_kernels.hpp).  A
// translation unit of its own so that it compiles in parallel with dQ.
#include "fa_bwd_kernels.hpp"

namespace fa {
namespace {

template <typename E, int D, bool CAUSAL, bool DROPOUT, bool CONTIG, bool SPLIT>
hipError_t launch_dkdv(BwdParams p, int heads, hipStream_t s) {
  p.num_blocks = (p.N + KvCfg<D>::BK - 1) / KvCfg<D>::BK;
  const int per_head = CAUSAL ? (p.num_blocks + 1) / 2 : p.num_blocks;
  p.units = heads * per_head * (SPLIT ? p.splits : 1);
  // Persistent grid: one workgroup per CU (each takes a whole CU's LDS and
  // registers), at most one per unit.
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int grid = p.units < cus ? p.units : cus;
  hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, CAUSAL, DROPOUT, CONTIG, SPLIT>), dim3(grid),
                     dim3(KvCfg<D>::THREADS), 0, s, p);
  return hipGetLastError();
}

// The split kernels exist for contiguous rows only.
template <typename E, int D, bool CONTIG, bool SPLIT>
hipError_t kv_flags(const BwdParams& p, bool causal, bool dropout, int heads, hipStream_t s) {
  if (causal)
    return dropout ? launch_dkdv<E, D, true, true, CONTIG, SPLIT>(p, heads, s)
                   : launch_dkdv<E, D, true, false, CONTIG, SPLIT>(p, heads, s);
  return dropout ? launch_dkdv<E, D, false, true, CONTIG, SPLIT>(p, heads, s)
                 : launch_dkdv<E, D, false, false, CONTIG, SPLIT>(p, heads, s);
}

template <typename E, int D>
hipError_t kv_d(const BwdParams& p, bool causal, bool dropout, bool contig, int heads, hipStream_t s) {
  if (p.splits > 0) {
    if (!contig) return hipErrorInvalidValue;
    return kv_flags<E, D, true, true>(p, causal, dropout, heads, s);
  }
  return contig ? kv_flags<E, D, true, false>(p, causal, dropout, heads, s)
                : kv_flags<E, D, false, false>(p, causal, dropout, heads, s);
}

}  // namespace

hipError_t launch_bwd_dkdv(BwdParams p, bool fp16, int d, bool causal, bool dropout, bool contig,
                           int heads, hipStream_t s) {
  if (fp16)
    return d == 64 ? kv_d<f16, 64>(p, causal, dropout, contig, heads, s)
                   : kv_d<f16, 128>(p, causal, dropout, contig, heads, s);
  return d == 64 ? kv_d<bf16, 64>(p, causal, dropout, contig, heads, s)
                 : kv_d<bf16, 128>(p, causal, dropout, contig, heads, s);
}

}  // namespace fa
