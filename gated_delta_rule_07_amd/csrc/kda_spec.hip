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
//   verify  the recurrence of section 3.3 of the technical report review,
//             Sbar_t = Diag(alpha_t) S_{t-1},  u_t = beta_t (v_t - Sbar_t^T k_t),
//             S_t = Sbar_t + k_t u_t^T,        o_t = S_t^T q_t,
//           unrolled over the draft.  With P_t = prod_{r<=t} alpha_r and
//           G_ts = prod_{s<r<=t} alpha_r (per key channel; tokens t = 0 .. K-1),
//             Sbar_t = Diag(P_t) S + sum_{s<t} Diag(G_ts) k_s u_s^T,
//           so every product with the state is one of 2K vectors,
//             x_t = S^T (P_t k_t) + sum_{s<t} c_ts u_s,   c_ts = sum_i k_s G_ts k_t,
//             u_t = beta_t (v_t - x_t),
//             o_t = S^T (P_t q_t) + sum_{s<t} d_ts u_s + d_tt u_t,
//                                                      d_ts = sum_i k_s G_ts q_t
//           (G_tt = 1).  S is read once and multiplied by all 2K vectors in one
//           pass; the K-step substitution then runs on each value column with
//           the scalars c and d, which depend only on k, q and alpha and are
//           formed while the state is in flight.  o_t and the write vectors
//           u_t are stored; S in memory is untouched.
//   commit  with j accepted tokens, the state after them has the closed form
//             S_j = Diag(P_j) S + sum_{t<j} Diag(P_j / P_{t+1}) k_t u_t^T,
//           P_m = prod_{s<m} alpha_s (per key channel),
//           which one streaming pass over S computes (j = 0 leaves S as it is).
//
// Both kernels: one workgroup per (sequence, head).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

// Commit: each thread owns a float4 column group and DK/RG rows.
template <int DK, int DV>
struct SCfg {
  static constexpr int NCG = DV / 4;                            // float4 column groups
  static constexpr int RG = (256 / NCG < DK) ? 256 / NCG : DK;  // row groups
  static constexpr int NT = NCG * RG;
  static constexpr int RPT = DK / RG;                           // rows per thread
  static constexpr int NW = NT / 64;
  static_assert(NT % 64 == 0 && NT <= 256, "block shape");
};

// Verify: wave w owns 4 CGW value columns of the state; lane (rg, cg) of it
// holds rows rg + RGW r (r < RPT) of its float4 column group, so a sum over the
// rows of the state is a sum within the wave.  A pass over the state forms the
// products with RGW vectors at a time, one per row-group lane after the sum.
template <int DK, int DV>
struct VCfg {
  static constexpr int CGW = DV >= 32 ? 8 : DV / 4;  // float4 column groups per wave
  static constexpr int RGW = 64 / CGW;               // row groups per wave = vectors per pass
  static constexpr int NW = DV / (4 * CGW);
  static constexpr int NT = 64 * NW;
  static constexpr int RPT = DK / RGW;                 // state rows per lane
  static constexpr int CPI = DK < 16 ? DK : 16;        // key channels per coefficient work item
  static constexpr int NCB = DK / CPI;
  static_assert(RPT >= 1 && DK % RGW == 0 && DV % (4 * CGW) == 0, "verify block shape");
};

// The verify kernel's LDS (floats, every region a multiple of 4), for K drafts.
// xs (the 2K state products) reuses the space of k, q and alpha, which are last
// read before it is written.
struct VLay {
  int nvp, np;                   // vectors padded to whole passes; token pairs s <= t
  int k, q, a, xs, v, b, pv, cp, dp, cc, dd, total;
  __host__ __device__ static int r4(int n) { return (n + 3) & ~3; }
  __host__ __device__ VLay(int K, int dk, int dv, int rgw, int ncb) {
    nvp = (2 * K + rgw - 1) / rgw * rgw;
    np = K * (K + 1) / 2;
    k = 0;
    q = k + r4(K * dk);
    a = q + r4(K * dk);
    xs = 0;
    int o = a + r4(K * dk);
    if (o < xs + nvp * dv) o = xs + nvp * dv;
    v = o;
    b = v + r4(K * dv);
    pv = b + r4(K);
    cp = pv + dk * nvp;
    dp = cp + r4(np * ncb);
    cc = dp + r4(np * ncb);
    dd = cc + r4(np);
    total = dd + r4(np);
  }
};

// Sums 2N vectors over lanes that differ in bit M and the bits below it down
// to the row-group bits: at each step a lane keeps half of its vectors (the
// upper half where its bit M is set) and adds its partner's copy of that half.
template <int N, int M>
__device__ __forceinline__ void reduce_scatter(f32x4* acc, int lane) {
  const bool up = (lane & M) != 0;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const f32x4 keep = up ? acc[N + e] : acc[e];
    const f32x4 send = up ? acc[e] : acc[N + e];
    f32x4 got;
#pragma unroll
    for (int c = 0; c < 4; ++c) got[c] = __shfl_xor(send[c], M);
    acc[e] = keep + got;
  }
  if constexpr (N > 1) reduce_scatter<N / 2, M / 2>(acc, lane);
}

__device__ __forceinline__ void block_sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename IO, int DK, int DV>
__global__ __launch_bounds__((VCfg<DK, DV>::NT)) void kda_verify_kernel(VerifyParams p) {
  using C = VCfg<DK, DV>;
  extern __shared__ f32x4 verify_lds[];
  float* sm = reinterpret_cast<float*>(verify_lds);
  const int K = p.K;
  const VLay L(K, DK, DV, C::RGW, C::NCB);
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int bh = blockIdx.x, b = bh / p.H, h = bh % p.H;
  const size_t row0 = (size_t)b * K * p.H + h;  // row (b, t, h) of the [B][K][H][d] inputs is row0 + t H

  // the drafts' keys, queries, decays, values and betas, then the state: all
  // loads in flight at once (small indices clamped into range, so no branch
  // splits them); storing the small ones to LDS waits only for them
  constexpr int EK = (kMaxDraft * DK + C::NT - 1) / C::NT, EV = (kMaxDraft * DV + C::NT - 1) / C::NT;
  const int nk = K * DK, nv = K * DV;
  IO rk[EK], rq[EK], rv[EV];
  float ra[EK];
#pragma unroll
  for (int j = 0; j < EK; ++j) {
    const int e = min(tid + j * C::NT, nk - 1);
    const size_t at = (row0 + (size_t)(e / DK) * p.H) * DK + e % DK;
    rk[j] = static_cast<const IO*>(p.k)[at];
    rq[j] = static_cast<const IO*>(p.q)[at];
    ra[j] = p.alpha[at];
  }
#pragma unroll
  for (int j = 0; j < EV; ++j) {
    const int e = min(tid + j * C::NT, nv - 1);
    rv[j] = static_cast<const IO*>(p.v)[(row0 + (size_t)(e / DV) * p.H) * DV + e % DV];
  }
  const float rb = p.beta[row0 + (size_t)min(tid, K - 1) * p.H];
  __builtin_amdgcn_sched_barrier(0);  // (the loads are counted in order: keep the small ones first)

  const int cg = lane % C::CGW, rg = lane / C::CGW;
  const int col = 4 * (C::CGW * wave + cg);
  f32x4 s[C::RPT];
  const float* S = p.S + (size_t)bh * DK * DV + col;
#pragma unroll
  for (int r = 0; r < C::RPT; ++r)
    s[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(rg + C::RGW * r) * DV));
  __builtin_amdgcn_sched_barrier(0);

  // (unconditional stores: a clamped index stores the value already there, and
  // no load is moved after the state's)
#pragma unroll
  for (int j = 0; j < EK; ++j) {
    const int e = min(tid + j * C::NT, nk - 1);
    sm[L.k + e] = to_f32(rk[j]);
    sm[L.q + e] = to_f32(rq[j]);
    sm[L.a + e] = ra[j];
  }
#pragma unroll
  for (int j = 0; j < EV; ++j) sm[L.v + min(tid + j * C::NT, nv - 1)] = to_f32(rv[j]);
  sm[L.b + min(tid, K - 1)] = rb;
  block_sync_lds();

  // while the state is in flight: the 2K vectors P_t k_t and P_t q_t, one key
  // channel per thread ...
  for (int i = tid; i < DK; i += C::NT) {
    float P = 1.0f;
    float* pv = sm + L.pv + i * L.nvp;
    for (int t = 0; t < K; ++t) {
      P *= sm[L.a + t * DK + i];
      pv[t] = P * sm[L.k + t * DK + i];
      pv[K + t] = P * sm[L.q + t * DK + i];
    }
    for (int j = 2 * K; j < L.nvp; ++j) pv[j] = 0.0f;
  }
  // ... and c_ts, d_ts for every pair s <= t, in partial sums over CPI channels
  for (int e = tid; e < L.np * C::NCB; e += C::NT) {
    const int pr = e / C::NCB, cb = e % C::NCB;
    int t = 0;
    while ((t + 1) * (t + 2) / 2 <= pr) ++t;
    const int s0 = pr - t * (t + 1) / 2;
    float cs = 0.0f, ds = 0.0f;
#pragma unroll 1
    for (int ii = 0; ii < C::CPI; ++ii) {
      const int i = cb + C::NCB * ii;
      float g = sm[L.k + s0 * DK + i];  // k_s G_ts
      for (int r = s0 + 1; r <= t; ++r) g *= sm[L.a + r * DK + i];
      cs += g * sm[L.k + t * DK + i];
      ds += g * sm[L.q + t * DK + i];
    }
    sm[L.cp + e] = cs;
    sm[L.dp + e] = ds;
  }
  block_sync_lds();
  for (int pr = tid; pr < L.np; pr += C::NT) {
    float cs = 0.0f, ds = 0.0f;
    for (int cb = 0; cb < C::NCB; ++cb) {
      cs += sm[L.cp + pr * C::NCB + cb];
      ds += sm[L.dp + pr * C::NCB + cb];
    }
    sm[L.cc + pr] = cs;
    sm[L.dd + pr] = ds;
  }

  // one pass over the state per RGW vectors: the lane's rows, then a
  // reduce-scatter over the row-group lanes, after which lane rg holds the sum
  // for vector g0 + rg
  for (int g0 = 0; g0 < L.nvp; g0 += C::RGW) {
    f32x4 acc[C::RGW];
#pragma unroll
    for (int j = 0; j < C::RGW; ++j) acc[j] = (f32x4)0.0f;
#pragma unroll
    for (int r = 0; r < C::RPT; ++r) {
      const float* pr = sm + L.pv + (rg + C::RGW * r) * L.nvp + g0;
#pragma unroll
      for (int j = 0; j < C::RGW; j += 4) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(pr + j);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[j + jj] += w[jj] * s[r];
      }
    }
    reduce_scatter<C::RGW / 2, 32>(acc, lane);
    *reinterpret_cast<f32x4*>(sm + L.xs + (g0 + rg) * DV + col) = acc[0];
  }
  block_sync_lds();

  // the substitution over the draft, one value column per thread
  if (tid < DV) {
    const int c = tid;
    float u[kMaxDraft];
#pragma unroll
    for (int t = 0; t < kMaxDraft; ++t) {
      if (t >= K) continue;
      const int pt = t * (t + 1) / 2;
      float x = sm[L.xs + t * DV + c];
      float y = sm[L.xs + (K + t) * DV + c];
#pragma unroll
      for (int s0 = 0; s0 < t; ++s0) {
        x += sm[L.cc + pt + s0] * u[s0];
        y += sm[L.dd + pt + s0] * u[s0];
      }
      u[t] = sm[L.b + t] * (sm[L.v + t * DV + c] - x);
      y += sm[L.dd + pt + t] * u[t];
      const size_t orow = row0 + (size_t)t * p.H;
      if (p.o_f32) static_cast<float*>(p.o)[orow * DV + c] = y;
      else static_cast<__bf16*>(p.o)[orow * DV + c] = (__bf16)y;
      p.u[((size_t)bh * K + t) * DV + c] = u[t];
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
  using C = VCfg<DK, DV>;
  const size_t lds = (size_t)VLay(p.K, DK, DV, C::RGW, C::NCB).total * sizeof(float);
  hipLaunchKernelGGL((kda_verify_kernel<IO, DK, DV>), dim3((unsigned)(p.B * p.H)), dim3(C::NT), lds, s, p);
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
