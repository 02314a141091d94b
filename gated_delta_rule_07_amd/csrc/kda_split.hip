// Sequence split for the prefill: the step between its two passes.
//
// Between chunks only the state travels (the "Kimi 모델 분석" write-up on
// rlaope.github.io, section on putting the recurrence on the GPU), and one token
// of the recurrence in section 3.3 of the "Kimi K3 Technical Report review"
// (jw9603.github.io), S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T, is
// affine in S_{t-1} with the same d_k x d_k matrix for every state column.  So
// is any run of tokens: the state after part j of a sequence is
// M_j S_in + N_j, with M_j the part's transition and N_j its state from zero.
// The first prefill pass computes (N_j | M_j) for every part but the last, the
// parts in parallel; this kernel chains them,
//     S_in(0) = S0,   S_in(j+1) = M_j S_in(j) + N_j,
// in fp32; the second pass reruns every part from S_in(j) (section 13 of the
// technical report review lists this kind of context parallelism).
//
// One workgroup per (b, h, 8 state columns): thread (r, half) owns row r and
// columns 4 half .. 4 half + 3; the current S_in slab lives in LDS.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

template <int DK>
__global__ __launch_bounds__(2 * DK) void kda_split_combine_kernel(PrefillParams p) {
  __shared__ f32x4 s[DK][2];
  const int tid = threadIdx.x;
  const int ng = p.dv / 8;
  const int g = blockIdx.x % ng, bh = blockIdx.x / ng;
  const int b = bh / p.H, h = bh % p.H;
  const int r = tid / 2, half = tid % 2;
  const int col = 8 * g + 4 * half;
  const size_t mat = (size_t)DK * p.dv;
  const int ld = p.dv + DK;  // row stride of (N | M)

  f32x4 cur = (f32x4)0.0f;
  if (p.S0) cur = *reinterpret_cast<const f32x4*>(p.S0 + (size_t)bh * mat + (size_t)r * p.dv + col);
  float* in0 = p.ws_in + ((size_t)(b * p.nparts) * p.H + h) * mat;
  *reinterpret_cast<f32x4*>(in0 + (size_t)r * p.dv + col) = cur;
  s[r][half] = cur;
  __syncthreads();
  for (int j = 0; j + 1 < p.nparts; ++j) {
    const float* tr = p.ws_trans + ((size_t)(b * (p.nparts - 1) + j) * p.H + h) * DK * ld + (size_t)r * ld;
    f32x4 acc = *reinterpret_cast<const f32x4*>(tr + col);  // N_j
    const float* m = tr + p.dv;                             // row r of M_j
#pragma unroll 4
    for (int k = 0; k < DK; k += 4) {
      const f32x4 mk = *reinterpret_cast<const f32x4*>(m + k);
      acc += mk[0] * s[k][half];
      acc += mk[1] * s[k + 1][half];
      acc += mk[2] * s[k + 2][half];
      acc += mk[3] * s[k + 3][half];
    }
    __syncthreads();  // every thread has read S_in(j)
    s[r][half] = acc;
    float* out = p.ws_in + ((size_t)(b * p.nparts + j + 1) * p.H + h) * mat;
    *reinterpret_cast<f32x4*>(out + (size_t)r * p.dv + col) = acc;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_split_combine(const PrefillParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)(p.B * p.H * (p.dv / 8));
  if (p.dk == 128) hipLaunchKernelGGL(kda_split_combine_kernel<128>, dim3(grid), dim3(256), 0, s, p);
  else if (p.dk == 64) hipLaunchKernelGGL(kda_split_combine_kernel<64>, dim3(grid), dim3(128), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kda
