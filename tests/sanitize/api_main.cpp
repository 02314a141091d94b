// Driver for the sanitizer build of the libkda C ABI (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code; the kernels are compiled for the
// host only, so no device code exists in this build and nothing can launch).
// It calls every entry point with arguments that validation must refuse, and
// the host-only planning queries with valid ones, and checks each status code;
// any invalid memory access or undefined behaviour in the validation and
// dispatch code aborts the run.  The pointers are fake, 16-byte aligned
// addresses that are never dereferenced.  Exit 0: clean.
#include <stdint.h>
#include <stdio.h>

#include "kda.h"

namespace {

int failures = 0;

void expect(const char* what, kda_status got, kda_status want) {
  if (got != want) {
    fprintf(stderr, "api sanitizer driver: %s returned %d, expected %d\n", what, (int)got, (int)want);
    ++failures;
  }
}

void* addr(int i, int off = 0) { return reinterpret_cast<void*>((uintptr_t(1) << 40) + (uintptr_t(i) << 32) + off); }
float* faddr(int i, int off = 0) { return static_cast<float*>(addr(i, off)); }

}  // namespace

int main() {
  const kda_dtype BF = KDA_BF16, F = KDA_F32;
  // prefill
  expect("prefill dtype", kda_chunk_fwd(addr(0), addr(1), addr(2), (kda_dtype)7, faddr(3), faddr(4), faddr(5), addr(6),
                                        F, faddr(7), 1, 64, 2, 128, 128, 64, nullptr), KDA_ERR_DTYPE);
  expect("prefill B", kda_chunk_fwd(addr(0), addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5), addr(6), F, faddr(7),
                                    0, 64, 2, 128, 128, 64, nullptr), KDA_ERR_SHAPE);
  expect("prefill d_k", kda_chunk_fwd(addr(0), addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5), addr(6), F,
                                      faddr(7), 1, 64, 2, 48, 128, 64, nullptr), KDA_ERR_UNSUPPORTED);
  expect("prefill chunk", kda_chunk_fwd(addr(0), addr(1), addr(2), F, faddr(3), faddr(4), faddr(5), addr(6), F,
                                        faddr(7), 1, 64, 2, 128, 128, 48, nullptr), KDA_ERR_UNSUPPORTED);
  expect("prefill null q", kda_chunk_fwd(nullptr, addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5), addr(6), F,
                                         faddr(7), 1, 64, 2, 128, 128, 64, nullptr), KDA_ERR_NULL);
  expect("prefill misaligned", kda_chunk_fwd(addr(0), addr(1, 8), addr(2), BF, faddr(3), faddr(4), faddr(5), addr(6),
                                             F, faddr(7), 1, 64, 2, 128, 128, 64, nullptr), KDA_ERR_MISALIGNED);
  expect("prefill alias", kda_chunk_fwd(addr(0), addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5), addr(0), F,
                                        faddr(7), 1, 64, 2, 128, 128, 64, nullptr), KDA_ERR_ALIAS);
  expect("prefill S_T overlaps S0", kda_chunk_fwd(addr(0), addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5),
                                                  addr(6), F, faddr(5, 16), 1, 64, 2, 128, 128, 64, nullptr),
         KDA_ERR_ALIAS);
  // snapshots
  const int bad_pos[2] = {64, 64};
  expect("snapshots order", kda_chunk_fwd_snapshots(addr(0), addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5),
                                                    addr(6), F, faddr(7), bad_pos, 2, faddr(8), 1, 300, 2, 128, 128,
                                                    64, nullptr), KDA_ERR_SHAPE);
  expect("snapshots count", kda_chunk_fwd_snapshots(addr(0), addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5),
                                                    addr(6), F, faddr(7), bad_pos, KDA_MAX_SNAPSHOTS + 1, faddr(8), 1,
                                                    300, 2, 128, 128, 64, nullptr), KDA_ERR_SHAPE);
  // varlen, gated, split
  expect("varlen offsets", kda_chunk_fwd_varlen(addr(0), addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5), addr(6),
                                                F, faddr(7), nullptr, 3, 300, 2, 128, 128, 64, nullptr), KDA_ERR_NULL);
  expect("varlen alias", kda_chunk_fwd_varlen(addr(0), addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5), addr(6), F,
                                              faddr(7), static_cast<const int*>(addr(6)), 3, 300, 2, 128, 128, 64,
                                              nullptr), KDA_ERR_ALIAS);
  expect("gated z", kda_chunk_fwd_gated(addr(0), addr(1), addr(2), BF, nullptr, faddr(9), faddr(4), faddr(5), addr(6),
                                        F, faddr(7), 1, 64, 2, 128, 128, 64, nullptr), KDA_ERR_NULL);
  expect("split workspace", kda_chunk_fwd_split(addr(0), addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5), addr(6),
                                                F, faddr(7), 1, 4096, 8, 128, 128, 64, 4, 256, nullptr, 0, nullptr),
         KDA_ERR_NULL);
  expect("split small workspace", kda_chunk_fwd_split(addr(0), addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5),
                                                      addr(6), F, faddr(7), 1, 4096, 8, 128, 128, 64, 4, 256,
                                                      addr(10), 64, nullptr), KDA_ERR_SHAPE);
  // decode, verify, commit
  expect("decode alias", kda_decode_step(addr(0), addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5), addr(5), F, 4, 2,
                                         128, 128, nullptr), KDA_ERR_ALIAS);
  expect("decode gated z", kda_decode_step_gated(addr(0), addr(1), addr(2), BF, nullptr, faddr(9), faddr(4), faddr(5),
                                                 addr(6), F, 4, 2, 128, 128, nullptr), KDA_ERR_NULL);
  expect("verify K", kda_decode_verify(addr(0), addr(1), addr(2), BF, faddr(3), faddr(4), faddr(5), addr(6), F,
                                       faddr(7), 4, KDA_MAX_DRAFT + 1, 2, 128, 128, nullptr), KDA_ERR_SHAPE);
  expect("commit alias", kda_decode_commit(addr(1), BF, faddr(3), faddr(7), static_cast<const int*>(addr(8)),
                                           faddr(7), 4, 4, 2, 128, 128, nullptr), KDA_ERR_ALIAS);
  // host-only planning queries over every size
  const int dims[4] = {16, 32, 64, 128}, chunks[3] = {16, 32, 64};
  for (int io = 0; io < 2; ++io)
    for (int dk : dims)
      for (int dv : dims)
        for (int c : chunks) {
          int run = 0, parts = 0;
          size_t ws = 0;
          expect("run chunk", kda_chunk_fwd_run_chunk((kda_dtype)io, 8, dk, dv, c, &run), KDA_OK);
          if (run != 16 && run != 32 && run != 64) ++failures;
          for (int P : {0, 1, 3, 40})
            expect("split plan", kda_chunk_fwd_split_plan((kda_dtype)io, 1, 4096, 8, dk, dv, c,
                                                          (io == 1 && dk >= 64 && dv % 32 == 0 && c >= 32) ? P : 1,
                                                          256, &parts, &ws), KDA_OK);
        }
  for (int s = -1; s < 10; ++s) (void)kda_status_string((kda_status)s);
  if (failures) {
    fprintf(stderr, "api sanitizer driver: %d failures\n", failures);
    return 1;
  }
  puts("api sanitizer driver: clean");
  return 0;
}
