// ladder.hip -- the first rung of the kernel ladder: shared-memory tiling with
// one output per lane.
//
// This is the structure of the kernel on the page "Shared Memory Tiling"
// (kernel listing and its "Key Mechanics"): a BLOCK x BLOCK tile of C per
// workgroup, one element per lane, BLOCK x BLOCK tiles of A and B staged in
// LDS by the whole workgroup, a barrier after the staging (no lane reads a
// tile before every lane has written it) and another after the dot product
// (no lane overwrites a tile another lane still reads).  With BLOCK = 32 the
// workgroup is 1024 lanes, i.e. 16 waves of 64.  Every load and store is
// masked, so any M, N, K and leading dimensions work.  It is a reference
// point for the tiled kernels, not a fast path: each loaded LDS value feeds
// a single FMA (the page's "two loads per FMA").
#include <hip/hip_runtime.h>

#include "sgemm_kernels.hpp"

namespace fp32gemm {

template <int BLOCK>
__global__ void __launch_bounds__(BLOCK * BLOCK) sgemm_smem_tiling_kernel(KernelArgs p) {
  __shared__ float As[BLOCK * BLOCK];
  __shared__ float Bs[BLOCK * BLOCK];
  const int tr = threadIdx.x / BLOCK, tc = threadIdx.x % BLOCK;
  const int row0 = (blockIdx.x / p.tiles_n) * BLOCK;
  const int col0 = (blockIdx.x % p.tiles_n) * BLOCK;
  const int r = row0 + tr, c = col0 + tc;
  float acc = 0.0f;
  for (int k0 = 0; k0 < p.K; k0 += BLOCK) {
    // Lane (tr, tc) stages A[r][k0 + tc] and B[k0 + tr][c]: a wave covers two
    // rows of 32 consecutive floats of each operand (coalesced).
    As[tr * BLOCK + tc] =
        (r < p.M && k0 + tc < p.K) ? p.A[static_cast<long long>(r) * p.lda + k0 + tc] : 0.0f;
    Bs[tr * BLOCK + tc] =
        (k0 + tr < p.K && c < p.N) ? p.B[static_cast<long long>(k0 + tr) * p.ldb + c] : 0.0f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BLOCK; ++k) acc = __builtin_fmaf(As[tr * BLOCK + k], Bs[k * BLOCK + tc], acc);
    __syncthreads();
  }
  if (r < p.M && c < p.N) {
    float* cp = p.C + static_cast<long long>(r) * p.ldc + c;
    float v = p.alpha * acc;
    if (p.beta != 0.0f) v = __builtin_fmaf(p.beta, *cp, v);
    *cp = v;
  }
}

hipError_t launch_smem_tiling(const KernelArgs& a, hipStream_t stream) {
  constexpr int kBlock = 32;
  KernelArgs k = a;
  const long long tiles_m = (a.M + kBlock - 1) / kBlock;
  const long long tiles_n = (a.N + kBlock - 1) / kBlock;
  if (tiles_m * tiles_n > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  k.tiles_m = static_cast<int>(tiles_m);
  k.tiles_n = static_cast<int>(tiles_n);
  void* args[] = {&k};
  return hipLaunchKernel(reinterpret_cast<const void*>(&sgemm_smem_tiling_kernel<kBlock>),
                         dim3(static_cast<unsigned>(tiles_m * tiles_n)), dim3(kBlock * kBlock), args,
                         0, stream);
}

}  // namespace fp32gemm
