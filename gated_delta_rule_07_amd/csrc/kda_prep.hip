// KDA prefill, stage 1 of 2: the chunk records of every (sequence, head,
// 32-token chunk) of a call or of one block of its chunks, one wave per record
// (the device code and the method are in kda_prep_impl.h).
#include "kda_prep_impl.h"

namespace kda {
namespace {

template <class C, bool G>
__global__ __launch_bounds__(64 * prep::kPrepWaves, 2) void kda_prep_kernel(PrefillParams p) {
  __shared__ prep::PrepLds<C> lds[prep::kPrepWaves];
  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  prep::prep_record<C, G>(p, (long long)blockIdx.x * prep::kPrepWaves + wave, lds[wave], lane);
}

template <int DK>
hipError_t launch_prep(const PrefillParams& p, long long nslots, hipStream_t s) {
  using C = prep::PCfg<DK>;
  const long long waves = nslots * p.H;
  const long long grid = (waves + prep::kPrepWaves - 1) / prep::kPrepWaves;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (p.z) hipLaunchKernelGGL((kda_prep_kernel<C, true>), dim3((unsigned)grid), dim3(64 * prep::kPrepWaves), 0, s, p);
  else hipLaunchKernelGGL((kda_prep_kernel<C, false>), dim3((unsigned)grid), dim3(64 * prep::kPrepWaves), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_prep(const PrefillParams& p, long long nslots, hipStream_t s) {
  if (p.dk == 128) return launch_prep<128>(p, nslots, s);
  if (p.dk == 64) return launch_prep<64>(p, nslots, s);
  return hipErrorInvalidValue;
}

}  // namespace kda
