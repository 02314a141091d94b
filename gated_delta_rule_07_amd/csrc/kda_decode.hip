// Batched KDA decode step for gfx950: one token per (sequence, head), state in place.
//
// One step of the recurrence of the "Kimi K3 Technical Report review"
// (jw9603.github.io, section 3.3, delta form):
//   Sbar = Diag(alpha) S,  x = Sbar^T k,  y = Sbar^T q,  d = beta (v - x),
//   S'   = Sbar + k d^T,   o = S'^T q = y + (k^T q) d.
// The last identity lets the readout be formed from the same pass over the
// state that forms x, so each fp32 state is read from HBM once and written once:
// decode is bound by those bytes ("Kimi 모델 분석", rlaope.github.io, section on
// why decoding is slow: arithmetic intensity far below the ridge, so the only
// lever is the bytes read per step).
//
// One workgroup per (sequence, head).  Each thread owns a float4 column group
// and DK/RG rows (interleaved, so one wave instruction covers whole 512-byte
// rows); the two reductions over rows run in registers, then across lanes with
// cross-lane shuffles and across waves through LDS.  No matrix cores: the
// products are matrix-vector shaped.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

template <int DK, int DV>
struct DCfg {
  static constexpr int NCG = DV / 4;                        // float4 column groups
  static constexpr int RG = (256 / NCG < DK) ? 256 / NCG : DK;  // row groups
  static constexpr int NT = NCG * RG;
  static constexpr int RPT = DK / RG;                       // rows per thread
  static constexpr int NW = NT / 64;
  static_assert(NT % 64 == 0 && NT <= 256, "decode block shape");
};

template <typename IO>
__device__ __forceinline__ void load4(const IO* p, float (&f)[4]);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float (&f)[4]) {
  const f32x4 w = *reinterpret_cast<const f32x4*>(p);
  f[0] = w.x; f[1] = w.y; f[2] = w.z; f[3] = w.w;
}
template <>
__device__ __forceinline__ void load4<__bf16>(const __bf16* p, float (&f)[4]) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  f[0] = __builtin_bit_cast(float, w.x << 16);
  f[1] = __builtin_bit_cast(float, w.x & 0xffff0000u);
  f[2] = __builtin_bit_cast(float, w.y << 16);
  f[3] = __builtin_bit_cast(float, w.y & 0xffff0000u);
}

template <typename IO>
__device__ __forceinline__ void store4(IO* p, const float (&f)[4]);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float (&f)[4]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* p, const float (&f)[4]) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 h;
  h[0] = (__bf16)f[0]; h[1] = (__bf16)f[1]; h[2] = (__bf16)f[2]; h[3] = (__bf16)f[3];
  *reinterpret_cast<bf16x4*>(p) = h;
}

template <typename IO, int DK, int DV>
__global__ __launch_bounds__(256) void kda_decode_kernel(DecodeParams p) {
  using C = DCfg<DK, DV>;
  __shared__ float sk[DK], sq[DK], sa[DK];
  __shared__ f32x4 sred[C::NW][C::NCG][2];
  __shared__ float skq[C::NW];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int cg = tid % C::NCG, rg = tid / C::NCG;
  const IO* q = static_cast<const IO*>(p.q) + (size_t)bh * DK;
  const IO* k = static_cast<const IO*>(p.k) + (size_t)bh * DK;
  const IO* v = static_cast<const IO*>(p.v) + (size_t)bh * DV;
  const float* alpha = p.alpha + (size_t)bh * DK;
  float* S = p.S + (size_t)bh * DK * DV;

  // Issue the state stream first: DK/RG float4 loads per thread, all independent.
  // Plain loads and non-temporal stores: measured on the B=256, H=32 workload,
  // this mix moves the state 9% faster than non-temporal loads as well (and 20%
  // faster than plain stores).
  f32x4 s[C::RPT];
#pragma unroll
  for (int r = 0; r < C::RPT; ++r) {
    const int i = rg + C::RG * r;
    s[r] = *reinterpret_cast<const f32x4*>(S + (size_t)i * DV + 4 * cg);
  }
  if (tid < DK) {
    sk[tid] = to_f32(k[tid]);
    sq[tid] = to_f32(q[tid]);
    // fused gate: alpha = exp(-5 sigmoid(e^A z)) from z in the q/k/v dtype
    sa[tid] = p.z ? gate_retention(__expf(p.A[bh % p.H]) * to_f32(static_cast<const IO*>(p.z)[(size_t)bh * DK + tid]))
                  : alpha[tid];
  }
  float vv[4];
  load4<IO>(v + 4 * cg, vv);
  const float beta = p.beta[bh];
  __syncthreads();

  // Decay rows, then the two row reductions x = Sbar^T k, y = Sbar^T q (and k^T q).
  f32x4 x = (f32x4)0.0f, y = (f32x4)0.0f;
  float kq = 0.0f;
#pragma unroll
  for (int r = 0; r < C::RPT; ++r) {
    const int i = rg + C::RG * r;
    const float ki = sk[i], qi = sq[i];
    s[r] *= sa[i];
    x += ki * s[r];
    y += qi * s[r];
    kq += ki * qi;
  }
#pragma unroll
  for (int off = C::NCG; off < 64; off *= 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] += __shfl_xor(x[e], off);
      y[e] += __shfl_xor(y[e], off);
    }
    kq += __shfl_xor(kq, off);
  }
  const int wave = tid / 64, lane = tid % 64;
  if (lane < C::NCG) {
    sred[wave][cg][0] = x;
    sred[wave][cg][1] = y;
    if (lane == 0) skq[wave] = kq;
  }
  __syncthreads();
  x = (f32x4)0.0f;
  y = (f32x4)0.0f;
  kq = 0.0f;
#pragma unroll
  for (int w = 0; w < C::NW; ++w) {
    x += sred[w][cg][0];
    y += sred[w][cg][1];
    kq += skq[w];
  }

  // d = beta (v - x); S' = Sbar + k d^T; o = y + (k^T q) d.
  f32x4 d;
#pragma unroll
  for (int e = 0; e < 4; ++e) d[e] = beta * (vv[e] - x[e]);
#pragma unroll
  for (int r = 0; r < C::RPT; ++r) {
    const int i = rg + C::RG * r;
    const f32x4 nv = s[r] + sk[i] * d;
    __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(S + (size_t)i * DV + 4 * cg));
  }
  if (rg == 0) {
    float ov[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ov[e] = y[e] + kq * d[e];
    if (p.o_f32) store4<float>(static_cast<float*>(p.o) + (size_t)bh * DV + 4 * cg, ov);
    else store4<__bf16>(static_cast<__bf16*>(p.o) + (size_t)bh * DV + 4 * cg, ov);
  }
}

template <typename IO, int DK, int DV>
hipError_t launch_one(const DecodeParams& p, hipStream_t s) {
  using C = DCfg<DK, DV>;
  hipLaunchKernelGGL((kda_decode_kernel<IO, DK, DV>), dim3((unsigned)(p.B * p.H)), dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

typedef hipError_t (*launch_fn)(const DecodeParams&, hipStream_t);

template <typename IO, int DK>
launch_fn pick_dv(int dv) {
  switch (dv) {
    case 16: return &launch_one<IO, DK, 16>;
    case 32: return &launch_one<IO, DK, 32>;
    case 64: return &launch_one<IO, DK, 64>;
    case 128: return &launch_one<IO, DK, 128>;
    default: return nullptr;
  }
}

template <typename IO>
launch_fn pick_dk(int dk, int dv) {
  switch (dk) {
    case 16: return pick_dv<IO, 16>(dv);
    case 32: return pick_dv<IO, 32>(dv);
    case 64: return pick_dv<IO, 64>(dv);
    case 128: return pick_dv<IO, 128>(dv);
    default: return nullptr;
  }
}

launch_fn pick(int io_dtype, int dk, int dv) {
  if (io_dtype == 1) return pick_dk<__bf16>(dk, dv);
  if (io_dtype == 0) return pick_dk<float>(dk, dv);
  return nullptr;
}

}  // namespace

bool decode_supported(int io_dtype, int dk, int dv) { return pick(io_dtype, dk, dv) != nullptr; }

hipError_t launch_decode(const DecodeParams& p, int io_dtype, hipStream_t s) {
  const launch_fn f = pick(io_dtype, p.dk, p.dv);
  if (!f) return hipErrorInvalidValue;
  return f(p, s);
}

}  // namespace kda
