// Load step (3) on the device: the layer's recovery basis.
//
// The down columns of every expert are stacked, D_all = [D_0 | ... | D_{E-1}]
// (H x E*I, not centred); U holds the top-`rank` left singular vectors and
// b_j = U^T d_j ([zh §前置知识 / 低秩恢复]; [zh §方法步骤详情] load step (3);
// [ko §어떻게 쓰나]; zh/ko = the Chinese/Korean summary pages of "Channel
// Selection for Mixture-of-Experts Decoding Needs No Calibration Data").
//
// The top eigenvalues of D_all D_all^T are close together (relative gaps of
// about 1e-3 for Gaussian weights), so the Gram is accumulated in float64
// here and handed to a full symmetric divide-and-conquer eigensolver
// (rocSOLVER dsyevd) rather than to a power iteration.  U and b are rounded
// to fp16 (nearest even) on the host.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <rocsolver/rocsolver.h>

#include <memory>
#include <vector>

#include "kernels.h"

namespace cfr {

namespace {

constexpr int kT = 64;   // Gram tile
constexpr int kNC = 32;  // channels per Gram step

__device__ __forceinline__ double bf16d(uint16_t b) {
  return (double)__uint_as_float((uint32_t)b << 16);
}

// Weight h of the down row of channel n in the [N][3] row layout (rows of
// rowq bytes): BF16, or a 4-bit record, scale (q - zero) (exact in double).
template <bool Q4>
__device__ __forceinline__ double down_w(const uint8_t* w3, size_t n, int h, int H, int rowq) {
  const uint8_t* row = w3 + (n * 3 + 2) * (size_t)rowq;
  if constexpr (Q4) {
    const int q = (row[h >> 1] >> (4 * (h & 1))) & 15;
    const uint16_t sb = *reinterpret_cast<const uint16_t*>(row + (H >> 1) + 2 * (h >> 7));
    const int z = row[(H >> 1) + (H >> 6) + (h >> 7)];
    return (double)__builtin_bit_cast(_Float16, sb) * (double)(q - z);
  } else {
    return bf16d(reinterpret_cast<const uint16_t*>(row)[h]);
  }
}

// G[i][j] = sum_n d_n[i] d_n[j] over all N channels, upper tiles only, mirrored.
// d_n is the transposed-down row of channel n inside the [N][3][H] layout.
template <bool Q4>
__global__ __launch_bounds__(256) void k_gram(const uint8_t* __restrict__ w3,
                                              double* __restrict__ G, int H, int N, int rowq) {
  const int tc = blockIdx.x, tr = blockIdx.y;
  if (tr > tc) return;
  __shared__ double A[kNC][kT];
  __shared__ double B[kNC][kT];
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  double acc[4][4] = {};
  for (int n0 = 0; n0 < N; n0 += kNC) {
    for (int q = tid; q < kNC * kT; q += 256) {
      const int nn = q / kT, h = q % kT, n = n0 + nn;
      A[nn][h] = n < N ? down_w<Q4>(w3, n, tr * kT + h, H, rowq) : 0.0;
      B[nn][h] = n < N ? down_w<Q4>(w3, n, tc * kT + h, H, rowq) : 0.0;
    }
    __syncthreads();
    for (int nn = 0; nn < kNC; ++nn) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = A[nn][ty * 4 + i];
        b[i] = B[nn][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = tr * kT + ty * 4 + i, c = tc * kT + tx * 4 + j;
      G[(size_t)r * H + c] = acc[i][j];
      G[(size_t)c * H + r] = acc[i][j];
    }
}

// b[n][r] = sum_h U[h][r] d_n[h]; eig holds eigenvectors as contiguous
// columns (column-major), ascending eigenvalue; column H-1-r is the r-th largest.
template <bool Q4>
__global__ __launch_bounds__(256) void k_coeffs(const uint8_t* __restrict__ w3,
                                                const double* __restrict__ eig,
                                                double* __restrict__ bout, int H, int N, int rank,
                                                int rowq) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)N * rank) return;
  const int n = (int)(idx / rank), r = (int)(idx % rank);
  const double* u = eig + (size_t)(H - 1 - r) * H;
  double acc = 0.0;
  for (int h = 0; h < H; ++h) acc += u[h] * down_w<Q4>(w3, n, h, H, rowq);
  bout[idx] = acc;
}

struct DevBuf {
  void* p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
};

}  // namespace

static int hipf(hipError_t e, const char* what) {
  return fail(CFR_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

int device_lowrank(cfr_reader* r) {
  const int H = r->cfg.hidden, rank = r->cfg.rank;
  const int N = r->cfg.n_experts * r->cfg.inter;
  if (rank == 0) return CFR_OK;
  DevBuf G, W, Eb, Info, Bb;
  hipError_t e;
  if ((e = hipMalloc(&G.p, sizeof(double) * H * H)) != hipSuccess ||
      (e = hipMalloc(&W.p, sizeof(double) * H)) != hipSuccess ||
      (e = hipMalloc(&Eb.p, sizeof(double) * H)) != hipSuccess ||
      (e = hipMalloc(&Info.p, sizeof(rocblas_int))) != hipSuccess ||
      (e = hipMalloc(&Bb.p, sizeof(double) * N * rank)) != hipSuccess)
    return fail(CFR_ENOMEM, std::string("lowrank workspace: ") + hipGetErrorString(e));
  const int nt = H / kT;
  const bool q4 = q4_rows(r->cfg);
  const int rowq = row_bytes(H, q4);
  if (q4)
    k_gram<true><<<dim3(nt, nt), 256>>>(r->w3, (double*)G.p, H, N, rowq);
  else
    k_gram<false><<<dim3(nt, nt), 256>>>(r->w3, (double*)G.p, H, N, rowq);
  if ((e = hipGetLastError()) != hipSuccess) return hipf(e, "gram launch");
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hipf(e, "gram");

  rocblas_handle h = nullptr;
  if (rocblas_create_handle(&h) != rocblas_status_success)
    return fail(CFR_ESOLVER, "rocblas_create_handle failed");
  rocblas_status st = rocsolver_dsyevd(h, rocblas_evect_original, rocblas_fill_upper, H,
                                       (double*)G.p, H, (double*)W.p, (double*)Eb.p,
                                       (rocblas_int*)Info.p);
  (void)hipDeviceSynchronize();
  rocblas_destroy_handle(h);
  if (st != rocblas_status_success) return fail(CFR_ESOLVER, "rocsolver_dsyevd failed");
  rocblas_int info = 0;
  if ((e = hipMemcpy(&info, Info.p, sizeof(info), hipMemcpyDeviceToHost)) != hipSuccess)
    return hipf(e, "eig info");
  if (info != 0) return fail(CFR_ESOLVER, "eigensolver did not converge (info != 0)");

  const long nb = (long)N * rank;
  if (q4)
    k_coeffs<true><<<(unsigned)((nb + 255) / 256), 256>>>(r->w3, (const double*)G.p, (double*)Bb.p, H, N,
                                                   rank, rowq);
  else
    k_coeffs<false><<<(unsigned)((nb + 255) / 256), 256>>>(r->w3, (const double*)G.p, (double*)Bb.p, H, N,
                                                   rank, rowq);
  if ((e = hipGetLastError()) != hipSuccess) return hipf(e, "coeffs launch");
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hipf(e, "coeffs");

  // fp16 rounding on the host
  std::vector<double> eig((size_t)rank * H), bh((size_t)nb);
  if ((e = hipMemcpy(eig.data(), (double*)G.p + (size_t)(H - rank) * H, sizeof(double) * rank * H,
                     hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(bh.data(), Bb.p, sizeof(double) * nb, hipMemcpyDeviceToHost)) != hipSuccess)
    return hipf(e, "lowrank download");
  std::vector<uint16_t> u16((size_t)H * rank), b16((size_t)nb);
  for (int rr = 0; rr < rank; ++rr) {
    const double* col = eig.data() + (size_t)(rank - 1 - rr) * H;  // (H-1-rr)-th column
    for (int hh = 0; hh < H; ++hh) u16[(size_t)hh * rank + rr] = f64_to_f16_rne(col[hh]);
  }
  for (long q = 0; q < nb; ++q) b16[q] = f64_to_f16_rne(bh[q]);
  if ((e = hipMemcpy(r->u, u16.data(), u16.size() * 2, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(r->b, b16.data(), b16.size() * 2, hipMemcpyHostToDevice)) != hipSuccess)
    return hipf(e, "lowrank upload");
  return CFR_OK;
}

}  // namespace cfr
