// Drives the host side of the library (argument checks, workspace plans,
// status strings, the measurement hook) with AddressSanitizer and
// UndefinedBehaviorSanitizer: csrc/bwattn.cpp is compiled for the host only
// and linked against the stand-in launchers below, which count calls and
// return an error without touching memory.  Valid calls stop at the device
// check (no GPU here), so no launcher is expected to run.  Prints
// "host checks ok" and exits 0 on success.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>

#include "bwattn.h"
#include "kernels.hpp"

static int g_launches = 0;

namespace bwattn {
#define STAND_IN(sig) \
  sig {               \
    ++g_launches;     \
    return hipErrorInvalidValue; \
  }
STAND_IN(hipError_t launch_packed_ce_prologue(const CeArgs&, hipStream_t))
STAND_IN(hipError_t launch_packed_ce_rows(const CeArgs&, hipStream_t))
STAND_IN(hipError_t launch_packed_ce_sum(const CeArgs&, hipStream_t))
STAND_IN(hipError_t launch_rope(const RopeArgs&, hipStream_t))
STAND_IN(hipError_t launch_rope_f32(const RopeArgs&, const float*, float*, hipStream_t))
STAND_IN(hipError_t launch_attn_fwd_f32(const F32Args&, int, hipStream_t))
STAND_IN(hipError_t launch_attn_bwd_dq_f32(const F32Args&, int, hipStream_t))
STAND_IN(hipError_t launch_attn_bwd_dkdv_f32(const F32Args&, int, hipStream_t))
STAND_IN(hipError_t launch_block_ranges(const int32_t*, int, int, int, int2*, hipStream_t))
STAND_IN(hipError_t launch_tile_ranges(const TileRangeArgs&, hipStream_t))
STAND_IN(hipError_t launch_tile64_ranges(const int2*, int, int, int, int, int2*, hipStream_t))
STAND_IN(hipError_t launch_attn_fwd(const FwdArgs&, int, hipStream_t))
STAND_IN(hipError_t launch_attn_bwd_dq(const BwdArgs&, int, hipStream_t))
STAND_IN(hipError_t launch_attn_bwd_dkdv(const BwdArgs&, int, hipStream_t))
STAND_IN(hipError_t launch_attn_decode_partial(const DecodeArgs&, int, hipStream_t))
STAND_IN(hipError_t launch_attn_decode_combine(const DecodeArgs&, int, hipStream_t))
STAND_IN(hipError_t decode_scratch(void**))
#undef STAND_IN
}  // namespace bwattn

static int g_fail = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "line %d: %s (last error: %s)\n", __LINE__, #cond, attn_last_error()); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

static attn_params params(int B, int H, int S, int D, double theta = 1e6, int kv_chunk = 0) {
  attn_params p;
  std::memset(&p, 0, sizeof(p));
  p.struct_size = (int32_t)sizeof(attn_params);
  p.batch = B;
  p.heads = H;
  p.seqlen = S;
  p.head_dim = D;
  p.causal = 1;
  p.rope_theta = theta;
  p.kv_chunk = kv_chunk;
  return p;
}

// distinct 16-byte aligned fake device addresses (never dereferenced)
static void* addr(int i) { return reinterpret_cast<void*>(static_cast<uintptr_t>(0x100000 + 256 * i)); }

int main() {
  // workspace plans over the whole parameter range, including the largest
  // sizes the checks admit (overflow checks under UBSan)
  const int dims[] = {64, 128};
  const int seqs[] = {1, 31, 32, 33, 255, 256, 1000, 65536, 1 << 20, 1 << 24};
  for (int D : dims)
    for (int S : seqs)
      for (int which = 0; which < 4; ++which) {
        attn_params p = params(1, 32, S, D, which & 1 ? 5e7 : 0.0);
        size_t ws = attn_workspace_bytes(&p, which);
        EXPECT(ws > 0);
      }
  {
    attn_params p = params(1 << 10, 1 << 10, 1 << 24, 128);
    EXPECT(attn_workspace_bytes(&p, 1) == 0);  // B*H*S*D above the limit
    p = params(1, 1, (1 << 24) + 1, 128);
    EXPECT(attn_workspace_bytes(&p, 0) == 0);
    p = params(1, 1, 64, 96);
    EXPECT(attn_workspace_bytes(&p, 0) == 0);
    p = params(1, 1, 64, 128);
    EXPECT(attn_workspace_bytes(&p, 4) == 0 && attn_workspace_bytes(&p, -1) == 0);
    EXPECT(attn_workspace_bytes(nullptr, 0) == 0);
  }
  // argument errors of every entry point come back before any HIP call
  attn_params ok = params(1, 2, 1024, 128);
  attn_params bad = ok;
  bad.struct_size = 8;
  const size_t big = attn_workspace_bytes(&ok, 1);
  EXPECT(attn_fwd(nullptr, addr(0), addr(1), addr(2), nullptr, nullptr, addr(3), (float*)addr(4), addr(5), big,
                  nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(attn_fwd(&bad, addr(0), addr(1), addr(2), nullptr, nullptr, addr(3), (float*)addr(4), addr(5), big,
                  nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(attn_fwd(&ok, (char*)addr(0) + 2, addr(1), addr(2), nullptr, nullptr, addr(3), (float*)addr(4), addr(5),
                  big, nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(attn_fwd(&ok, addr(0), addr(1), addr(2), nullptr, nullptr, addr(3), (float*)addr(4), addr(5), 16,
                  nullptr) == ATTN_ERR_WORKSPACE);
  EXPECT(attn_bwd(&ok, addr(0), addr(1), addr(2), addr(3), nullptr, addr(4), nullptr, nullptr, addr(5), addr(6),
                  addr(7), addr(8), big, nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(attn_bwd(&ok, addr(0), addr(1), addr(2), addr(3), (float*)addr(9), addr(4), nullptr, nullptr, addr(5),
                  addr(6), addr(7), nullptr, 0, nullptr) == ATTN_ERR_WORKSPACE);
  EXPECT(attn_fwd_f32(&ok, nullptr, (float*)addr(1), (float*)addr(2), nullptr, nullptr, (float*)addr(3),
                      (float*)addr(4), addr(5), big, nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(attn_bwd_f32(&bad, (float*)addr(0), (float*)addr(1), (float*)addr(2), (float*)addr(3), (float*)addr(9),
                      (float*)addr(4), nullptr, nullptr, (float*)addr(5), (float*)addr(6), (float*)addr(7), addr(8),
                      big, nullptr) == ATTN_ERR_INVALID_ARG);
  attn_params notheta = params(1, 2, 64, 64, 0.0);
  EXPECT(rope_apply(&notheta, addr(0), addr(1), nullptr, 0, nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(rope_apply(&ok, addr(0), addr(1), nullptr, 5, nullptr) == ATTN_ERR_INVALID_ARG);
  EXPECT(rope_apply_f32(&ok, nullptr, (float*)addr(1), nullptr, 0, nullptr) == ATTN_ERR_INVALID_ARG);
  attn_params chunk = params(1, 2, 1024, 128, 1e6, 100);
  EXPECT(attn_fwd(&chunk, addr(0), addr(1), addr(2), nullptr, nullptr, addr(3), (float*)addr(4), addr(5), big,
                  nullptr) == ATTN_ERR_INVALID_ARG);
  // decode
  EXPECT(attn_decode_workspace_bytes(&ok, 0) == 0 && attn_decode_workspace_bytes(&ok, 33) == 0);
  const size_t dws = attn_decode_workspace_bytes(&ok, 4);
  EXPECT(dws > 0);
  EXPECT(attn_decode(&ok, 4, addr(0), addr(1), addr(2), nullptr, addr(3), (float*)addr(4), addr(5), dws - 1,
                     nullptr) == ATTN_ERR_WORKSPACE);
  EXPECT(attn_decode(&ok, 2000, addr(0), addr(1), addr(2), nullptr, addr(3), (float*)addr(4), addr(5), dws,
                     nullptr) == ATTN_ERR_INVALID_ARG);
  // decode without a workspace: parameters beyond the static workspace are
  // refused before any HIP call
  EXPECT(attn_decode_noalloc_max_bytes() == (size_t(64) << 20));
  attn_params wide = params(64, 64, 1024, 128);  // 4096 heads x 32 rows: about 96 MiB
  EXPECT(attn_decode_workspace_bytes(&wide, 32) > attn_decode_noalloc_max_bytes());
  EXPECT(attn_decode_noalloc(&wide, 32, addr(0), addr(1), addr(2), nullptr, addr(3), (float*)addr(4), nullptr) ==
         ATTN_ERR_WORKSPACE);
  EXPECT(attn_decode_noalloc(&ok, 0, addr(0), addr(1), addr(2), nullptr, addr(3), (float*)addr(4), nullptr) ==
         ATTN_ERR_INVALID_ARG);
  EXPECT(attn_decode_noalloc(&ok, 4, addr(0), nullptr, addr(2), nullptr, addr(3), (float*)addr(4), nullptr) ==
         ATTN_ERR_INVALID_ARG);
  // packed cross-entropy
  packed_ce_params cp;
  std::memset(&cp, 0, sizeof(cp));
  cp.struct_size = (int32_t)sizeof(cp);
  cp.batch = 1;
  cp.seqlen = 4096;
  cp.vocab = 40192;
  cp.num_segments = 7;
  cp.grad_scale = 1.f;
  const size_t cws = packed_ce_workspace_bytes(&cp);
  EXPECT(cws > 0);
  EXPECT(packed_ce_loss(&cp, addr(0), (int32_t*)addr(1), nullptr, (float*)addr(2), addr(3), nullptr, addr(4), 8,
                        nullptr) == ATTN_ERR_WORKSPACE);
  packed_ce_params cbad = cp;
  cbad.vocab = 65544;
  EXPECT(packed_ce_workspace_bytes(&cbad) == 0);
  cbad = cp;
  cbad.vocab = 12;
  EXPECT(packed_ce_loss(&cbad, addr(0), (int32_t*)addr(1), nullptr, (float*)addr(2), addr(3), nullptr, addr(4),
                        cws, nullptr) == ATTN_ERR_INVALID_ARG);
  // valid calls stop at the device check: no GPU in this process
  int rc = attn_fwd(&ok, addr(0), addr(1), addr(2), nullptr, nullptr, addr(3), (float*)addr(4), addr(5), big,
                    nullptr);
  EXPECT(rc == ATTN_ERR_HIP || rc == ATTN_ERR_UNSUPPORTED);
  EXPECT(std::strlen(attn_last_error()) > 0);
  // measurement hook and status strings
  EXPECT(attn_profile_events(ATTN_KERNEL_COUNT, nullptr, nullptr, 0) == ATTN_ERR_INVALID_ARG);
  EXPECT(attn_profile_events(ATTN_KERNEL_FWD, nullptr, nullptr, 3) == ATTN_ERR_INVALID_ARG);
  EXPECT(attn_profile_events(ATTN_KERNEL_FWD, nullptr, nullptr, 0) == ATTN_OK);
  EXPECT(attn_profile_count(-1) == -1 && attn_profile_count(ATTN_KERNEL_FWD) == 0);
  for (int s = -1; s < 6; ++s) EXPECT(attn_status_string(s) != nullptr);
  EXPECT(g_launches == 0);
  if (g_fail) {
    std::fprintf(stderr, "%d host checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks ok\n");
  return 0;
}
