// Speculative decoding for KDA on gfx950: verify K draft tokens without
// touching the state, then commit the accepted prefix.
//
// A KDA layer keeps one state per (sequence, head) and each decode step
// overwrites it, so the tokens a draft model proposed cannot simply be cut off
// again when the target model rejects them (the "Kimi 모델 분석" write-up on
// rlaope.github.io, serving section, on speculative decoding; the "Kimi K3
// Technical Report review" on jw9603.github.io, section 13, lists restoring the
// state after rejected draft tokens).  Here the K tokens are split in two passes
// over the state:
//
//   verify  S is read once and the recurrence of section 3.3 of the technical
//           report review is applied to K tokens in registers:
//             Sbar = Diag(alpha_t) S,  x = Sbar^T k_t,  u_t = beta_t (v_t - x),
//             S <- Sbar + k_t u_t^T,   o_t = S^T q_t = Sbar^T q_t + (k_t^T q_t) u_t.
//           o_t and the write vectors u_t are stored; S in memory is untouched.
//   commit  with j accepted tokens, the state after them has the closed form
//             S_j = Diag(P_j) S + sum_{t<j} Diag(P_j / P_{t+1}) k_t u_t^T,
//           P_m = prod_{s<m} alpha_s (per key channel),
//           which one streaming pass over S computes (j = 0 leaves S as it is).
//
// Both kernels: one workgroup per (sequence, head); each thread owns a float4
// column group and DK/RG rows, as in the single-token decode kernel.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

template <int DK, int DV>
struct SCfg {
  static constexpr int NCG = DV / 4;                            // float4 column groups
  static constexpr int RG = (256 / NCG < DK) ? 256 / NCG : DK;  // row groups
  static constexpr int NT = NCG * RG;
  static constexpr int RPT = DK / RG;                           // rows per thread
  static constexpr int NW = NT / 64;
  static_assert(NT % 64 == 0 && NT <= 256, "block shape");
};

__device__ __forceinline__ void load4(const float* p, f32x4& f) { f = *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void load4(const __bf16* p, f32x4& f) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  f = f32x4{__builtin_bit_cast(float, w.x << 16), __builtin_bit_cast(float, w.x & 0xffff0000u),
            __builtin_bit_cast(float, w.y << 16), __builtin_bit_cast(float, w.y & 0xffff0000u)};
}

__device__ __forceinline__ void store_o(void* o, size_t idx, const f32x4& f, int o_f32) {
  if (o_f32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(o) + idx) = f;
  } else {
    typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
    const bf16x4v h = {(__bf16)f[0], (__bf16)f[1], (__bf16)f[2], (__bf16)f[3]};
    *reinterpret_cast<bf16x4v*>(static_cast<__bf16*>(o) + idx) = h;
  }
}

template <typename IO, int DK, int DV>
__global__ __launch_bounds__(256) void kda_verify_kernel(VerifyParams p) {
  using C = SCfg<DK, DV>;
  __shared__ float sk[kMaxDraft][DK], sq[kMaxDraft][DK], sa[kMaxDraft][DK];
  __shared__ f32x4 sred[2][C::NW][C::NCG][2];  // per token parity: no barrier before reuse
  __shared__ float skq[2][C::NW];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x, b = bh / p.H, h = bh % p.H;
  const int cg = tid % C::NCG, rg = tid / C::NCG;
  const int wave = tid / 64, lane = tid % 64;
  const int K = p.K;

  f32x4 s[C::RPT];
  const float* S = p.S + (size_t)bh * DK * DV;
#pragma unroll
  for (int r = 0; r < C::RPT; ++r)
    s[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(rg + C::RG * r) * DV + 4 * cg));
  // the K tokens' keys, queries and decays (row (b, t, h) of the [B][K][H][d] inputs)
  for (int e = tid; e < K * DK; e += C::NT) {
    const int t = e / DK, i = e % DK;
    const size_t row = ((size_t)b * K + t) * p.H + h;
    sk[t][i] = to_f32(static_cast<const IO*>(p.k)[row * DK + i]);
    sq[t][i] = to_f32(static_cast<const IO*>(p.q)[row * DK + i]);
    sa[t][i] = p.alpha[row * DK + i];
  }
  __syncthreads();

  for (int t = 0; t < K; ++t) {
    const size_t row = ((size_t)b * K + t) * p.H + h;
    f32x4 vv;
    load4(static_cast<const IO*>(p.v) + row * DV + 4 * cg, vv);
    const float beta = p.beta[row];
    f32x4 x = (f32x4)0.0f, y = (f32x4)0.0f;
    float kq = 0.0f;
#pragma unroll
    for (int r = 0; r < C::RPT; ++r) {
      const int i = rg + C::RG * r;
      const float ki = sk[t][i], qi = sq[t][i];
      s[r] *= sa[t][i];
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
    const int par = t & 1;
    if (lane < C::NCG) {
      sred[par][wave][cg][0] = x;
      sred[par][wave][cg][1] = y;
      if (lane == 0) skq[par][wave] = kq;
    }
    __syncthreads();
    x = (f32x4)0.0f;
    y = (f32x4)0.0f;
    kq = 0.0f;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) {
      x += sred[par][w][cg][0];
      y += sred[par][w][cg][1];
      kq += skq[par][w];
    }
    const f32x4 d = beta * (vv - x);
#pragma unroll
    for (int r = 0; r < C::RPT; ++r) s[r] += sk[t][rg + C::RG * r] * d;
    if (rg == 0) {
      store_o(p.o, row * DV + 4 * cg, y + kq * d, p.o_f32);
      *reinterpret_cast<f32x4*>(p.u + ((size_t)bh * K + t) * DV + 4 * cg) = d;
    }
  }
}

template <typename IO, int DK, int DV>
__global__ __launch_bounds__(256) void kda_commit_kernel(CommitParams p) {
  using C = SCfg<DK, DV>;
  __shared__ float coef[kMaxDraft][DK];  // k_t * P_j / P_{t+1}
  __shared__ float pj[DK];               // P_j
  const int tid = threadIdx.x;
  const int bh = blockIdx.x, b = bh / p.H, h = bh % p.H;
  const int cg = tid % C::NCG, rg = tid / C::NCG;
  const int K = p.K;
  const int j = min(max(p.n_accept[b], 0), K);
  if (j == 0) return;  // nothing accepted: the state stays as it is

  float* S = p.S + (size_t)bh * DK * DV;
  // plain loads with the non-temporal stores below: faster than non-temporal both ways
  f32x4 s[C::RPT];
#pragma unroll
  for (int r = 0; r < C::RPT; ++r) s[r] = *reinterpret_cast<const f32x4*>(S + (size_t)(rg + C::RG * r) * DV + 4 * cg);
  for (int i = tid; i < DK; i += C::NT) {
    float run = 1.0f;  // product of the decays after token t
    for (int t = j - 1; t >= 0; --t) {
      const size_t row = ((size_t)b * K + t) * p.H + h;
      coef[t][i] = to_f32(static_cast<const IO*>(p.k)[row * DK + i]) * run;
      run *= p.alpha[row * DK + i];
    }
    pj[i] = run;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < C::RPT; ++r) s[r] *= pj[rg + C::RG * r];
  for (int t = 0; t < j; ++t) {
    const f32x4 ut = *reinterpret_cast<const f32x4*>(p.u + ((size_t)bh * K + t) * DV + 4 * cg);
#pragma unroll
    for (int r = 0; r < C::RPT; ++r) s[r] += coef[t][rg + C::RG * r] * ut;
  }
#pragma unroll
  for (int r = 0; r < C::RPT; ++r)
    __builtin_nontemporal_store(s[r], reinterpret_cast<f32x4*>(S + (size_t)(rg + C::RG * r) * DV + 4 * cg));
}

template <typename IO, int DK, int DV>
hipError_t verify_one(const VerifyParams& p, hipStream_t s) {
  hipLaunchKernelGGL((kda_verify_kernel<IO, DK, DV>), dim3((unsigned)(p.B * p.H)), dim3(SCfg<DK, DV>::NT), 0, s, p);
  return hipGetLastError();
}
template <typename IO, int DK, int DV>
hipError_t commit_one(const CommitParams& p, hipStream_t s) {
  hipLaunchKernelGGL((kda_commit_kernel<IO, DK, DV>), dim3((unsigned)(p.B * p.H)), dim3(SCfg<DK, DV>::NT), 0, s, p);
  return hipGetLastError();
}

template <class P>
using spec_fn = hipError_t (*)(const P&, hipStream_t);

template <typename IO, int DK, int DV>
struct VerifyF {
  static constexpr spec_fn<VerifyParams> fn = &verify_one<IO, DK, DV>;
};
template <typename IO, int DK, int DV>
struct CommitF {
  static constexpr spec_fn<CommitParams> fn = &commit_one<IO, DK, DV>;
};

template <class P, template <typename, int, int> class F, typename IO, int DK>
spec_fn<P> pick_dv(int dv) {
  switch (dv) {
    case 16: return F<IO, DK, 16>::fn;
    case 32: return F<IO, DK, 32>::fn;
    case 64: return F<IO, DK, 64>::fn;
    case 128: return F<IO, DK, 128>::fn;
    default: return nullptr;
  }
}

template <class P, template <typename, int, int> class F, typename IO>
spec_fn<P> pick_dk(int dk, int dv) {
  switch (dk) {
    case 16: return pick_dv<P, F, IO, 16>(dv);
    case 32: return pick_dv<P, F, IO, 32>(dv);
    case 64: return pick_dv<P, F, IO, 64>(dv);
    case 128: return pick_dv<P, F, IO, 128>(dv);
    default: return nullptr;
  }
}

template <class P, template <typename, int, int> class F>
spec_fn<P> pick(int io_dtype, int dk, int dv) {
  if (io_dtype == 1) return pick_dk<P, F, __bf16>(dk, dv);
  if (io_dtype == 0) return pick_dk<P, F, float>(dk, dv);
  return nullptr;
}

}  // namespace

bool spec_supported(int io_dtype, int dk, int dv) {
  return pick<VerifyParams, VerifyF>(io_dtype, dk, dv) != nullptr;
}

hipError_t launch_verify(const VerifyParams& p, int io_dtype, hipStream_t s) {
  const spec_fn<VerifyParams> f = pick<VerifyParams, VerifyF>(io_dtype, p.dk, p.dv);
  if (!f || p.K < 1 || p.K > kMaxDraft) return hipErrorInvalidValue;
  return f(p, s);
}

hipError_t launch_commit(const CommitParams& p, int io_dtype, hipStream_t s) {
  const spec_fn<CommitParams> f = pick<CommitParams, CommitF>(io_dtype, p.dk, p.dv);
  if (!f || p.K < 1 || p.K > kMaxDraft) return hipErrorInvalidValue;
  return f(p, s);
}

}  // namespace kda
