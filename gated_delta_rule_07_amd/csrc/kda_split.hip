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
// One workgroup per (b, h, 4 state columns), KQ * DK threads: thread (r, kq)
// owns row r and the kq-th of KQ key ranges of the product (the ranges are
// summed with lane shuffles).  The parts are sequential, so the latency of each
// part is what counts: the rows of M and N for part j + 2 are loaded while part
// j is multiplied (three register buffers, rotated by unrolling), and the
// current S_in slab sits in LDS, double-buffered so each part takes one barrier.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int KQ = 8;  // key ranges per row

template <int DK>
__global__ __launch_bounds__(KQ * DK) void kda_split_combine_kernel(PrefillParams p) {
  constexpr int KR = DK / KQ;  // keys per thread
  constexpr int NL = KR / 4;   // float4 loads of M per thread and part
  __shared__ f32x4 s[2][DK];
  const int tid = threadIdx.x;
  const int kq = tid % KQ, r = tid / KQ;
  const int ng = p.dv / 4;
  const int g = blockIdx.x % ng, bh = blockIdx.x / ng;
  const int b = bh / p.H, h = bh % p.H;
  const int col = 4 * g;
  const int P = p.nparts;
  const size_t mat = (size_t)DK * p.dv;
  const int ld = p.dv + DK;  // row stride of (N | M)
  auto trans = [&](int j) {  // row r of (N_j | M_j)
    return p.ws_trans + ((size_t)(b * (P - 1) + j) * p.H + h) * DK * ld + (size_t)r * ld;
  };
  auto slot = [&](int j) { return p.ws_in + ((size_t)(b * P + j) * p.H + h) * mat + (size_t)r * p.dv + col; };
  // Rows of M_j (this thread's keys) and of N_j.  Loads, stores and LDS writes
  // are unconditional (part indices clamped, every lane of a row storing the
  // same value), so the compiler can count the loads still in flight and wait
  // only for the oldest buffer instead of for all of them.
  auto load = [&](int j, f32x4 (&m)[NL], f32x4& n) {
    const float* tr = trans(min(j, P - 2));
#pragma unroll
    for (int i = 0; i < NL; ++i) m[i] = *reinterpret_cast<const f32x4*>(tr + p.dv + kq * KR + 4 * i);
    n = *reinterpret_cast<const f32x4*>(tr + col);
  };
  // S_in(j+1) = M_j S_in(j) + N_j, prefetching part j + 2 into (mp, np)
  auto part = [&](int j, const f32x4 (&m)[NL], const f32x4& n, f32x4 (&mp)[NL], f32x4& np) {
    load(j + 2, mp, np);
    const f32x4* sj = s[j & 1];
    f32x4 acc = kq == 0 ? n : (f32x4)0.0f;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int k = kq * KR + 4 * i;
      acc += m[i][0] * sj[k];
      acc += m[i][1] * sj[k + 1];
      acc += m[i][2] * sj[k + 2];
      acc += m[i][3] * sj[k + 3];
    }
#pragma unroll
    for (int off = 1; off < KQ; off *= 2)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], off);
    s[(j + 1) & 1][r] = acc;  // the same value from every lane of row r
    *reinterpret_cast<f32x4*>(slot(j + 1)) = acc;
    __syncthreads();  // S_in(j+1) visible; every read of the other buffer is done
  };

  f32x4 cur = (f32x4)0.0f;
  if (p.S0) cur = *reinterpret_cast<const f32x4*>(p.S0 + (size_t)bh * mat + (size_t)r * p.dv + col);
  *reinterpret_cast<f32x4*>(slot(0)) = cur;
  s[0][r] = cur;
  f32x4 m0[NL], m1[NL], m2[NL], n0, n1, n2;
  load(0, m0, n0);
  load(1, m1, n1);
  __syncthreads();
  for (int j = 0; j + 1 < P; j += 3) {
    part(j, m0, n0, m2, n2);
    if (j + 2 >= P) break;
    part(j + 1, m1, n1, m0, n0);
    if (j + 3 >= P) break;
    part(j + 2, m2, n2, m1, n1);
  }
}

}  // namespace

hipError_t launch_split_combine(const PrefillParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)(p.B * p.H * (p.dv / 4));
  if (p.dk == 128) hipLaunchKernelGGL(kda_split_combine_kernel<128>, dim3(grid), dim3(KQ * 128), 0, s, p);
  else if (p.dk == 64) hipLaunchKernelGGL(kda_split_combine_kernel<64>, dim3(grid), dim3(KQ * 64), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kda
