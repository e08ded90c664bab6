// dQ and per-row-term launchers of the backward pass (kernels in
// fa_bwd_kernels.hpp).  A translation unit of its own so that it compiles
// in parallel with the dK/dV kernels.
#include "fa_bwd_kernels.hpp"

namespace fa {
namespace {

template <typename E, int D, bool CAUSAL, bool DROPOUT, bool CONTIG, bool SPLIT>
hipError_t launch_dq(BwdParams p, int heads, hipStream_t s) {
  p.num_blocks = (p.N + QCfg<D>::BM - 1) / QCfg<D>::BM;
  const int per_head = CAUSAL ? (p.num_blocks + 1) / 2 : p.num_blocks;
  const int64_t grid = (int64_t)heads * per_head * (SPLIT ? p.splits : 1);
  hipLaunchKernelGGL((bwd_dq_kernel<E, D, CAUSAL, DROPOUT, CONTIG, SPLIT>), dim3((unsigned)grid),
                     dim3(QCfg<D>::THREADS), 0, s, p);
  return hipGetLastError();
}

// The split kernels exist for contiguous rows only.
template <typename E, int D, bool CONTIG, bool SPLIT>
hipError_t dq_flags(const BwdParams& p, bool causal, bool dropout, int heads, hipStream_t s) {
  if (causal)
    return dropout ? launch_dq<E, D, true, true, CONTIG, SPLIT>(p, heads, s)
                   : launch_dq<E, D, true, false, CONTIG, SPLIT>(p, heads, s);
  return dropout ? launch_dq<E, D, false, true, CONTIG, SPLIT>(p, heads, s)
                 : launch_dq<E, D, false, false, CONTIG, SPLIT>(p, heads, s);
}

template <typename E, int D>
hipError_t dq_d(const BwdParams& p, bool causal, bool dropout, bool contig, int heads, hipStream_t s) {
  if (p.splits > 0) {
    if (!contig) return hipErrorInvalidValue;
    return dq_flags<E, D, true, true>(p, causal, dropout, heads, s);
  }
  return contig ? dq_flags<E, D, true, false>(p, causal, dropout, heads, s)
                : dq_flags<E, D, false, false>(p, causal, dropout, heads, s);
}

template <typename E, int D>
hipError_t pre_d(const BwdParams& p, int64_t rows, hipStream_t s) {
  const int64_t threads = rows * (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<E, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     p, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pre(const BwdParams& p, bool fp16, int d, int64_t rows, hipStream_t s) {
  if (fp16) return d == 64 ? pre_d<f16, 64>(p, rows, s) : pre_d<f16, 128>(p, rows, s);
  return d == 64 ? pre_d<bf16, 64>(p, rows, s) : pre_d<bf16, 128>(p, rows, s);
}

hipError_t launch_bwd_dq(BwdParams p, bool fp16, int d, bool causal, bool dropout, bool contig,
                         int heads, hipStream_t s) {
  if (fp16)
    return d == 64 ? dq_d<f16, 64>(p, causal, dropout, contig, heads, s)
                   : dq_d<f16, 128>(p, causal, dropout, contig, heads, s);
  return d == 64 ? dq_d<bf16, 64>(p, causal, dropout, contig, heads, s)
                 : dq_d<bf16, 128>(p, causal, dropout, contig, heads, s);
}

}  // namespace fa
