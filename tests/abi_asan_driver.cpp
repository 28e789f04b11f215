// Host-side driver for the C ABI of libattn (include/attn.h), built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code by
// tests/test_abi_asan.py.  It needs no GPU: every call either fails argument
// validation (and must return the documented status without touching any
// pointer) or reaches the device check, which fails with ATTN_ERR_DEVICE on
// a machine without a GPU.  Prints one line per failed expectation and
// returns the number of failures.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "attn.h"

namespace {

int g_fail = 0;

void expect(const char* what, long long got, long long want) {
  if (got != want) {
    std::printf("FAIL %s: got %lld, want %lld\n", what, got, want);
    ++g_fail;
  }
}

// Fake, 16-byte aligned device addresses: never dereferenced on these paths.
void* const A = reinterpret_cast<void*>(0x10000);
void* const U = reinterpret_cast<void*>(0x10008);  // misaligned
float* const F = reinterpret_cast<float*>(0x10000);

size_t stws_big() { return ~(size_t)0; }

}  // namespace

int main() {
  // forward
  expect("fwd null q", attn_fwd(nullptr, A, A, A, F, 1, 128, 2, 2, 64, 1, 0, 0.125f, nullptr), ATTN_ERR_NULLPTR);
  expect("fwd shape", attn_fwd(A, A, A, A, F, 1, 128, 4, 3, 64, 1, 0, 0.125f, nullptr), ATTN_ERR_SHAPE);
  expect("fwd head dim", attn_fwd(A, A, A, A, F, 1, 128, 2, 2, 96, 1, 0, 0.125f, nullptr), ATTN_ERR_HEADDIM);
  expect("fwd dtype", attn_fwd(A, A, A, A, F, 1, 128, 2, 2, 64, 7, 0, 0.125f, nullptr), ATTN_ERR_DTYPE);
  expect("fwd align", attn_fwd(A, U, A, A, F, 1, 128, 2, 2, 64, 1, 0, 0.125f, nullptr), ATTN_ERR_ALIGN);
  expect("fwd scale", attn_fwd(A, A, A, A, F, 1, 128, 2, 2, 64, 1, 0, NAN, nullptr), ATTN_ERR_SCALE);
  expect("fwd too large", attn_fwd(A, A, A, A, F, 1, 1 << 24, 1, 1, 128, 1, 0, 0.125f, nullptr),
         ATTN_ERR_TOO_LARGE);
  expect("fwd int overflow", attn_fwd(A, A, A, A, F, 0x7fffffff, 0x7fffffff, 0x7fffffff, 1, 256, 1, 0, 0.1f,
                                      nullptr), ATTN_ERR_TOO_LARGE);
  // backward and its stages
  const size_t ws = attn_bwd_workspace_bytes(1, 128, 2, 2, 64);
  expect("bwd workspace bytes", (long long)ws, 1 * 2 * 128 * 4);
  expect("bwd workspace invalid", (long long)attn_bwd_workspace_bytes(1, 16, 3, 2, 64), 0);
  expect("bwd workspace huge", (long long)attn_bwd_workspace_bytes(0x7fffffff, 0x7fffffff, 1, 1, 64), 0);
  expect("bwd null dk", attn_bwd(A, A, A, A, A, F, A, nullptr, A, A, ws, 1, 128, 2, 2, 64, 1, 0, 0.125f, nullptr),
         ATTN_ERR_NULLPTR);
  expect("bwd small workspace",
         attn_bwd(A, A, A, A, A, F, A, A, A, A, ws - 1, 1, 128, 2, 2, 64, 1, 0, 0.125f, nullptr), ATTN_ERR_WORKSPACE);
  expect("bwd_dkdv null workspace",
         attn_bwd_dkdv(A, A, A, A, A, F, A, A, A, nullptr, ws, 1, 128, 2, 2, 64, 1, 0, 0.125f, nullptr),
         ATTN_ERR_WORKSPACE);
  expect("bwd_dq align", attn_bwd_dq(A, A, A, A, A, F, U, A, A, A, ws, 1, 128, 2, 2, 64, 1, 0, 0.125f, nullptr),
         ATTN_ERR_ALIGN);
  expect("bwd_preprocess scale",
         attn_bwd_preprocess(A, A, A, A, A, F, A, A, A, A, ws, 1, 128, 2, 2, 64, 1, 0, INFINITY, nullptr),
         ATTN_ERR_SCALE);
  // rectangular and split-KV
  expect("fwd_rect shape", attn_fwd_rect(A, A, A, A, F, 1, 128, 0, 2, 2, 64, 1, 1, 0, 0.125f, nullptr),
         ATTN_ERR_SHAPE);
  expect("bwd_rect workspace", attn_bwd_rect(A, A, A, A, A, F, A, A, A, A, 0, 1, 128, 256, 2, 2, 64, 1, 1,
                                             -(1LL << 40), 0.125f, nullptr), ATTN_ERR_WORKSPACE);
  const size_t sws = attn_fwd_splitkv_workspace_bytes(1, 128, 2, 64, 4);
  expect("splitkv workspace bytes nonzero", sws > 0, 1);
  expect("splitkv workspace too large", (long long)attn_fwd_splitkv_workspace_bytes(0x7fffffff, 0x7fffffff, 0x7fffffff,
                                                                                  256, 256), 0);
  expect("standard int overflow", attn_fwd_standard(A, A, A, A, F, A, stws_big(), 0x7fffffff, 0x7fffffff, 0x7fffffff,
                                                    1, 64, 1, 1, 0.125f, nullptr), ATTN_ERR_TOO_LARGE);
  expect("splitkv splits", attn_fwd_splitkv(A, A, A, A, F, A, sws, 1, 128, 1000, 2, 2, 64, 1, 0, 0, 0.125f, 0,
                                            nullptr), ATTN_ERR_SHAPE);
  expect("splitkv small workspace", attn_fwd_splitkv(A, A, A, A, F, A, sws - 1, 1, 128, 1000, 2, 2, 64, 1, 0, 0,
                                                     0.125f, 4, nullptr), ATTN_ERR_WORKSPACE);
  // block-sparse
  const unsigned char* M = reinterpret_cast<const unsigned char*>(A);
  expect("sparse null mask", attn_fwd_blocksparse(A, A, A, A, F, nullptr, 1, 1, 128, 2, 2, 64, 1, 0, 0.125f,
                                                  nullptr), ATTN_ERR_NULLPTR);
  expect("sparse mask heads", attn_bwd_blocksparse(A, A, A, A, A, F, M, 3, A, A, A, A, ws, 1, 128, 2, 2, 64, 1, 0,
                                                   0.125f, nullptr), ATTN_ERR_SHAPE);
  // standard attention
  const size_t stws = attn_standard_workspace_bytes(1, 100, 2, 1, 64);
  expect("standard workspace bytes", (long long)stws, 4LL * 2 * 100 * 128 + 2 * (2LL * 2 * 100 * 128));
  expect("standard workspace too large", (long long)attn_standard_workspace_bytes(1, 1 << 20, 32, 32, 64), 0);
  expect("standard fwd workspace", attn_fwd_standard(A, A, A, A, F, A, stws - 1, 1, 100, 2, 1, 64, 1, 1, 0.125f,
                                                     nullptr), ATTN_ERR_WORKSPACE);
  expect("standard bwd null", attn_bwd_standard(A, A, A, nullptr, A, A, A, A, stws, 1, 100, 2, 1, 64, 1, 1,
                                                0.125f, nullptr), ATTN_ERR_NULLPTR);
  // status strings
  for (int s = 0; s <= ATTN_ERR_TOO_LARGE; ++s) {
    const char* m = attn_strerror(s);
    expect("strerror known", m != nullptr && std::strcmp(m, "unknown status") != 0, 1);
  }
  expect("strerror unknown", std::strcmp(attn_strerror(-5), "unknown status"), 0);
  expect("version", std::strstr(attn_version(), "gfx950") != nullptr, 1);
  // a valid call reaches the device check: no GPU here
  expect("valid call without a GPU", attn_fwd(A, A, A, A, F, 1, 128, 2, 2, 64, 1, 0, 0.125f, nullptr),
         ATTN_ERR_DEVICE);
  std::printf("%d failures\n", g_fail);
  return g_fail;
}
