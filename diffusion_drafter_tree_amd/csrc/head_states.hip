// Step a0 of the synthetic head: h[m][j] = sum_i H[m][i] * P[i][j], the
// per-position head input built from the drafter's shared representation H_d
// (marsggbo blog, section 3.1: one block-parallel forward gives H_d and the
// base logits). P is stored output-major: Pt[j][i] = P[i][j].
//
// bf16 path: one 256-thread workgroup per 16x16 output tile, the four waves
// split the D reduction (v_mfma_f32_16x16x32_bf16: bf16 x bf16 products are
// exact, accumulation in fp32) and their partial tiles are added in a fixed
// order, so results are reproducible run to run. fp32 path: one thread per
// output, plain fp32 fused multiply-adds.
#include "common.h"
#include "kernels.h"

namespace dartree {

namespace {

__global__ __launch_bounds__(256) void head_states_mfma(const uint16_t* __restrict__ H,
                                                        const uint16_t* __restrict__ Pt, float* __restrict__ h, int M,
                                                        int D, int r) {
  __shared__ float part[4][16][17];
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int nt = blockIdx.x, mt = blockIdx.y;
  const int ksteps = D / 32;
  const int k0 = (ksteps * w) / 4, k1 = (ksteps * (w + 1)) / 4;
  const int m = mt * 16 + (lane & 15);
  const int n = nt * 16 + (lane & 15);
  const int sub = (lane >> 4) * 8;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* hrow = H + (size_t)(m < M ? m : 0) * D;
  const uint16_t* prow = Pt + (size_t)n * D;
  for (int ks = k0; ks < k1; ++ks) {
    u16x8_t a = *reinterpret_cast<const u16x8_t*>(hrow + ks * 32 + sub);
    u16x8_t b = *reinterpret_cast<const u16x8_t*>(prow + ks * 32 + sub);
    if (m >= M) a = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    acc = mfma_bf16(a, b, acc);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[w][(lane >> 4) * 4 + i][lane & 15] = acc[i];
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = (lane >> 4) * 4 + i, cc = lane & 15;
      float v = ((part[0][rr][cc] + part[1][rr][cc]) + part[2][rr][cc]) + part[3][rr][cc];
      const int mm = mt * 16 + rr;
      if (mm < M) h[(size_t)mm * r + nt * 16 + cc] = v;
    }
  }
}

template <typename T>
__device__ __forceinline__ float ld_w(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld_w<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_w<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

template <typename T>
__global__ __launch_bounds__(256) void head_states_valu(const T* __restrict__ H, const T* __restrict__ Pt,
                                                        float* __restrict__ h, int M, int D, int r) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)M * r) return;
  const int m = (int)(idx / r), j = (int)(idx % r);
  float acc = 0.f;
  for (int i = 0; i < D; ++i) acc = fmaf(ld_w(H, (size_t)m * D + i), ld_w(Pt, (size_t)j * D + i), acc);
  h[idx] = acc;
}

}  // namespace

hipError_t launch_head_states(bool bf16, const void* H, const void* Pt, float* h, int M, int D, int r,
                              hipStream_t s) {
  const bool mfma_ok = bf16 && (D % 32 == 0) && (r % 16 == 0) && (((uintptr_t)H | (uintptr_t)Pt) & 15u) == 0;
  if (mfma_ok) {
    dim3 grid(r / 16, (M + 15) / 16);
    hipLaunchKernelGGL(head_states_mfma, grid, dim3(256), 0, s, static_cast<const uint16_t*>(H),
                       static_cast<const uint16_t*>(Pt), h, M, D, r);
  } else {
    const size_t total = (size_t)M * r;
    dim3 grid((unsigned)((total + 255) / 256));
    if (bf16)
      hipLaunchKernelGGL(head_states_valu<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(H),
                         static_cast<const uint16_t*>(Pt), h, M, D, r);
    else
      hipLaunchKernelGGL(head_states_valu<float>, grid, dim3(256), 0, s, static_cast<const float*>(H),
                         static_cast<const float*>(Pt), h, M, D, r);
  }
  return hipGetLastError();
}

}  // namespace dartree
