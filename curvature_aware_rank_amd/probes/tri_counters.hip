// Counter driver: one tridiagonalisation of a random symmetric 4096 x 4096 matrix (the
// library's own source) plus a plain copy kernel
// of known size (256 MiB), for rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE) whose
// copy-kernel reading calibrates the symv kernel's.  Build (from the repository root):
//   hipcc -O3 -std=c++17 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//     -I include -I curvature_aware_rank_amd/csrc curvature_aware_rank_amd/probes/tri_counters.hip \
//     curvature_aware_rank_amd/csrc/lrc_common.hip curvature_aware_rank_amd/csrc/lrc_dense.hip \
//     -o curvature_aware_rank_amd/probes/tri_counters
#include "../csrc/lrc_tridiag.hip"
#include <stdio.h>
#include <vector>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)
__global__ void copy_f4_kernel(const float4* __restrict__ s, float4* __restrict__ d, int64_t n4) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += int64_t(gridDim.x) * blockDim.x)
    d[i] = s[i];
}
int main() {
  const int n = 4096;
  const int64_t lda = n;
  using namespace lrc;
  double* A;
  CK(hipMalloc(&A, sizeof(double) * lda * n));
  {
    std::vector<double> h(size_t(lda) * n, 0.0);
    srand(7);
    for (int r = 0; r < n; ++r)
      for (int c = 0; c <= r; ++c) {
        const double v = double(rand()) / RAND_MAX - 0.5 + (r == c ? 4.0 : 0.0);
        h[size_t(r) * lda + c] = v;
        h[size_t(c) * lda + r] = v;
      }
    CK(hipMemcpy(A, h.data(), h.size() * 8, hipMemcpyHostToDevice));
  }
  void* ws;
  CK(hipMalloc(&ws, tridiag_workspace(n, 1024)));
  Carve cv(ws);
  TWs w = carve_tri(cv, n, 1024);
  hipStream_t st;
  CK(hipStreamCreate(&st));
  // copy of 256 MiB (known bytes: 256 MiB read, 256 MiB written)
  const int64_t nbytes = int64_t(256) << 20;
  float4 *s4, *d4;
  CK(hipMalloc(&s4, nbytes));
  CK(hipMalloc(&d4, nbytes));
  CK(hipMemsetAsync(s4, 1, nbytes, st));
  copy_f4_kernel<<<4096, 256, 0, st>>>(s4, d4, nbytes / 16);
  CK(hipGetLastError());
  if (tri_reduce(st, A, n, lda, w) != LRC_OK) { printf("tri_reduce failed\n"); return 1; }
  CK(hipStreamSynchronize(st));
  printf("done\n");
  return 0;
}
