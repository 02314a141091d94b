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
// parts in parallel; the kernels here form
//     S_in(0) = S0,   S_in(j+1) = M_j S_in(j) + N_j,
// in fp32, as a chain below kTreeParts parts and as a tree over the part maps
// from there on (below); the second pass reruns every part from S_in(j)
// (section 13 of the technical report review lists this kind of context
// parallelism).
//
// The chain: one workgroup per (b, h, 4 state columns), KQ * DK threads: thread (r, kq)
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

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
  // Part addresses are uniform (a buffer resource per part) and each thread's
  // offsets are fixed, so a part needs no vector address arithmetic: computed
  // per part, it landed in registers still awaiting the previous prefetch, and
  // the compiler waited for that prefetch at the start of every part.
  const int vo_m = 4 * (r * ld + p.dv + kq * KR);  // this thread's keys of row r of M_j
  const int vo_n = 4 * (r * ld + col);             // row r, this slab's columns, of N_j
  const int vo_s = 4 * (r * p.dv + col);           // the same in S_in(j)
  auto trans = [&](int j) {  // (N_j | M_j)
    return make_rsrc(p.ws_trans + ((size_t)(b * (P - 1) + j) * p.H + h) * DK * ld, DK * ld * 4);
  };
  auto slot = [&](int j) { return make_rsrc(p.ws_in + ((size_t)(b * P + j) * p.H + h) * mat, (int)(mat * 4)); };
  // Rows of M_j (this thread's keys) and of N_j.  Loads, stores and LDS writes
  // are unconditional (part indices clamped, every lane of a row storing the
  // same value), so the compiler can count the loads still in flight and wait
  // only for the oldest buffer instead of for all of them.
  auto load = [&](int j, f32x4 (&m)[NL], f32x4& n) {
    const __amdgpu_buffer_rsrc_t tr = trans(min(j, P - 2));
#pragma unroll
    for (int i = 0; i < NL; ++i) m[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, vo_m, 16 * i, 0));
    n = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, vo_n, 0, 0));
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
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), slot(j + 1), vo_s, 0, 0);
    __syncthreads();  // S_in(j+1) visible; every read of the other buffer is done
  };

  f32x4 cur = (f32x4)0.0f;
  if (p.S0) cur = *reinterpret_cast<const f32x4*>(p.S0 + (size_t)bh * mat + (size_t)r * p.dv + col);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, cur), slot(0), vo_s, 0, 0);
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


// ---- tree combine ----------------------------------------------------------
// For many parts the chain above is a long sequence of dependent steps.  The
// part maps compose associatively, (M_a, N_a) o (M_b, N_b) = (M_a M_b,
// M_a N_b + N_a), so an inclusive scan over them takes log2(P - 1) levels: at
// level d every part j >= d becomes its composition with part j - d (both from
// the previous level), parts j < d are carried over.  Afterwards part j holds
// the map of parts 0..j together, and S_in(j + 1) = M*_j S0 + N*_j.
//
// Both kernels compute DK x 32 tiles of M X in fp32: one 256-thread workgroup
// per (b, h, part, 32-column block).  M and X's column block pass through LDS
// TK keys at a time (row-major, 16-byte writes); the next phase's values are
// loaded into registers while the current phase is multiplied, so only the
// first phase's loads are waited for.
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int TC = 32;  // output columns per workgroup
constexpr int TNT = 256;
constexpr int TK = 32;  // keys per phase

template <int DK>
struct TilePhase {
  static constexpr int NA = DK * TK / 4 / TNT;  // f32x4 of M per thread and phase
  static constexpr int NX = TK * TC / 4 / TNT;  // f32x4 of X per thread and phase (1)
  static_assert(NA >= 1 && NX == 1, "tile phase shape");
  f32x4 a[NA];
  f32x4 x;
};

template <int DK>
__device__ __forceinline__ void tile_load(TilePhase<DK>& t, const float* M, int ldm, const float* X, int ldx, int kb,
                                          int tid) {
#pragma unroll
  for (int n = 0; n < TilePhase<DK>::NA; ++n) {
    const int e = tid + n * TNT, row = e / (TK / 4), k4 = 4 * (e % (TK / 4));
    t.a[n] = *reinterpret_cast<const f32x4*>(M + (size_t)row * ldm + kb + k4);
  }
  const int k = tid / (TC / 4), c4 = tid % (TC / 4);
  t.x = *reinterpret_cast<const f32x4*>(X + (size_t)(kb + k) * ldx + 4 * c4);
}

template <int DK>
__device__ __forceinline__ void tile_store(const TilePhase<DK>& t, float (&am)[DK][TK + 4], f32x4 (&xs)[TK][TC / 4],
                                           int tid) {
#pragma unroll
  for (int n = 0; n < TilePhase<DK>::NA; ++n) {
    const int e = tid + n * TNT, row = e / (TK / 4), k4 = 4 * (e % (TK / 4));
    *reinterpret_cast<f32x4*>(&am[row][k4]) = t.a[n];
  }
  xs[tid / (TC / 4)][tid % (TC / 4)] = t.x;
}

// The 32-row block 32 w.. of M X for wave w (row stride ldm of M, ldx of X, X
// offset to the tile's columns) on fp32 matrix cores: 32 x 32 x 2 steps, lane
// l supplying M[32 w + l % 32][k + l / 32] and X[k + l / 32][l % 32]; the
// result holds rows 8 (e / 4) + 4 (l / 32) + e % 4 of column l % 32 in element
// e.  fp32 products and sums throughout, at twice the unpacked vector rate.
// Waves whose block lies past DK return zeros.  LDS is reusable on return.
template <int DK>
__device__ __forceinline__ f32x16 tile_mfma(float (&am)[DK][TK + 4], f32x4 (&xs)[TK][TC / 4], const float* M, int ldm,
                                            const float* X, int ldx, int tid) {
  const int wave = tid / 64, lane = tid % 64, i = lane % 32, hk = lane / 32;
  const int row = 32 * wave + i;
  f32x16 d = (f32x16)0.0f;
  TilePhase<DK> t;
  tile_load<DK>(t, M, ldm, X, ldx, 0, tid);
  for (int kb = 0; kb < DK; kb += TK) {
    tile_store<DK>(t, am, xs, tid);
    __syncthreads();
    if (kb + TK < DK) tile_load<DK>(t, M, ldm, X, ldx, kb + TK, tid);  // in flight during the products
    if (32 * wave < DK) {
#pragma unroll
      for (int k = 0; k < TK; k += 2) {
        const float av = am[row][k + hk];
        const float bv = reinterpret_cast<const float*>(&xs[k + hk][0])[i];
        d = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, d, 0, 0, 0);
      }
    }
    __syncthreads();
  }
  return d;
}

// One level: dst_j = src_j o src_{j-d} for j >= d, dst_j = src_j for j < d, on
// (N | M) blocks of ld = dv + DK columns.
template <int DK>
__global__ __launch_bounds__(TNT) void kda_split_level_kernel(PrefillParams p, const float* src, float* dst, int d) {
  __shared__ float am[DK][TK + 4];
  __shared__ f32x4 xs[TK][TC / 4];
  const int ld = p.dv + DK, ncb = ld / TC, np = p.nparts - 1;
  const int cb = blockIdx.x % ncb, j = (blockIdx.x / ncb) % np, bh = blockIdx.x / ncb / np;
  const int b = bh / p.H, h = bh % p.H;
  const size_t blk = (size_t)DK * ld;
  auto part = [&](const float* base, int jj) { return base + ((size_t)(b * np + jj) * p.H + h) * blk; };
  const int tid = threadIdx.x;
  const float* sj = part(src, j);
  float* dj = const_cast<float*>(part(dst, j));
  const int col = cb * TC;
  if (j < d) {  // carried over
    for (int e = tid; e < DK * TC / 4; e += TNT) {
      const int r = e / (TC / 4), c4 = e % (TC / 4);
      *reinterpret_cast<f32x4*>(dj + (size_t)r * ld + col + 4 * c4) =
          *reinterpret_cast<const f32x4*>(sj + (size_t)r * ld + col + 4 * c4);
    }
    return;
  }
  // M_j X_{j-d} over this column block, plus N_j in the N columns
  const f32x16 acc = tile_mfma<DK>(am, xs, sj + p.dv, ld, part(src, j - d) + col, ld, tid);
  const int wave = tid / 64, lane = tid % 64;
  if (32 * wave < DK) {
    const int c = col + lane % 32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const size_t o = (size_t)(32 * wave + 8 * (e / 4) + 4 * (lane / 32) + e % 4) * ld + c;
      dj[o] = acc[e] + (col < p.dv ? sj[o] : 0.0f);
    }
  }
}

// S_in(0) = S0 (zeros when null), S_in(j+1) = M*_j S0 + N*_j.
template <int DK>
__global__ __launch_bounds__(TNT) void kda_split_apply_kernel(PrefillParams p, const float* comp) {
  __shared__ float am[DK][TK + 4];
  __shared__ f32x4 xs[TK][TC / 4];
  const int ld = p.dv + DK, ncb = p.dv / TC, P = p.nparts;
  const int cb = blockIdx.x % ncb, j = (blockIdx.x / ncb) % P, bh = blockIdx.x / ncb / P;
  const int b = bh / p.H, h = bh % p.H;
  const int tid = threadIdx.x;
  const size_t mat = (size_t)DK * p.dv;
  const int col = cb * TC;
  float* out = p.ws_in + ((size_t)(b * P + j) * p.H + h) * mat + col;
  const float* s0 = p.S0 ? p.S0 + (size_t)bh * mat + col : nullptr;
  const float* cj = j > 0 ? comp + ((size_t)(b * (P - 1) + j - 1) * p.H + h) * DK * ld : nullptr;
  if (j == 0 || !s0) {  // S0 itself, or N*_{j-1} alone
    for (int e = tid; e < DK * TC / 4; e += TNT) {
      const int r = e / (TC / 4), c4 = e % (TC / 4);
      f32x4 v = (f32x4)0.0f;
      if (j == 0 && s0) v = *reinterpret_cast<const f32x4*>(s0 + (size_t)r * p.dv + 4 * c4);
      if (j > 0) v = *reinterpret_cast<const f32x4*>(cj + (size_t)r * ld + col + 4 * c4);
      *reinterpret_cast<f32x4*>(out + (size_t)r * p.dv + 4 * c4) = v;
    }
    return;
  }
  const f32x16 acc = tile_mfma<DK>(am, xs, cj + p.dv, ld, s0, p.dv, tid);
  const int wave = tid / 64, lane = tid % 64;
  if (32 * wave < DK) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const size_t r = 32 * wave + 8 * (e / 4) + 4 * (lane / 32) + e % 4;
      out[r * p.dv + lane % 32] = acc[e] + cj[r * ld + col + lane % 32];
    }
  }
}

template <int DK>
hipError_t launch_tree(const PrefillParams& p, hipStream_t s) {
  const int np = p.nparts - 1, ld = p.dv + DK;
  const unsigned lgrid = (unsigned)(p.B * p.H * np * (ld / TC));
  float* src = p.ws_trans;
  float* dst = p.ws_tree;
  for (int d = 1; d < np; d *= 2) {
    hipLaunchKernelGGL(kda_split_level_kernel<DK>, dim3(lgrid), dim3(TNT), 0, s, p, (const float*)src, dst, d);
    float* t = src;
    src = dst;
    dst = t;
  }
  const unsigned agrid = (unsigned)(p.B * p.H * p.nparts * (p.dv / TC));
  hipLaunchKernelGGL(kda_split_apply_kernel<DK>, dim3(agrid), dim3(TNT), 0, s, p, (const float*)src);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split_combine(const PrefillParams& p, hipStream_t s) {
  if (p.nparts >= kTreeParts) {
    if (!p.ws_tree) return hipErrorInvalidValue;
    if (p.dk == 128) return launch_tree<128>(p, s);
    if (p.dk == 64) return launch_tree<64>(p, s);
    return hipErrorInvalidValue;
  }
  const unsigned grid = (unsigned)(p.B * p.H * (p.dv / 4));
  if (p.dk == 128) hipLaunchKernelGGL(kda_split_combine_kernel<128>, dim3(grid), dim3(KQ * 128), 0, s, p);
  else if (p.dk == 64) hipLaunchKernelGGL(kda_split_combine_kernel<64>, dim3(grid), dim3(KQ * 64), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kda
