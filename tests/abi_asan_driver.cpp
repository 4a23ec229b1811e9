// Host-only driver for the C ABI, built with AddressSanitizer on the host
// code (tests/test_abi_asan.py).  Every call below is refused by host-side
// validation before any HIP call, so it runs without a GPU; the point is that
// the validation and error-reporting code of every entry point stays inside
// its memory.  Prints one line per mismatch and exits with their count.
#include <cstdio>
#include <cstring>

#include "tokengate.h"

namespace {

int g_bad = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("MISMATCH %s: got %d want %d (%s)\n", what, got, want, tg_last_error());
    ++g_bad;
  }
  // The message of the last call is a valid C string of bounded length.
  const char* msg = tg_last_error();
  if (msg == nullptr || std::strlen(msg) >= 512) {
    std::printf("BAD MESSAGE after %s\n", what);
    ++g_bad;
  }
}

}  // namespace

int main() {
  void* F = reinterpret_cast<void*>(0x10000);  // 16-byte aligned, never dereferenced
  void* M = reinterpret_cast<void*>(0x10004);  // misaligned
  const float* Ff = static_cast<const float*>(F);
  const int32_t* Fi = static_cast<const int32_t*>(F);
  int32_t* Fo = static_cast<int32_t*>(F);
  float* Fw = static_cast<float*>(F);
  const int IA = TG_ERR_INVALID_ARG, UN = TG_ERR_UNSUPPORTED, WS = TG_ERR_WORKSPACE;

  // gate
  expect(tg_gate_score((tg_dtype)7, 10, 64, 64, F, 64, F, nullptr, Ff, 0.f, Fw, nullptr, nullptr), IA, "gate dtype");
  expect(tg_gate_score(TG_BF16, -1, 64, 64, F, 64, F, nullptr, Ff, 0.f, Fw, nullptr, nullptr), IA, "gate n");
  expect(tg_gate_score(TG_BF16, 10, 100, 64, F, 104, F, nullptr, Ff, 0.f, Fw, nullptr, nullptr), UN, "gate d");
  expect(tg_gate_score(TG_BF16, 10, 64, 96, F, 64, F, nullptr, Ff, 0.f, Fw, nullptr, nullptr), UN, "gate hidden");
  expect(tg_gate_score(TG_BF16, 10, 64, 64, M, 64, F, nullptr, Ff, 0.f, Fw, nullptr, nullptr), IA, "gate align");
  expect(tg_gate_score(TG_FP32, 1 << 26, 4, 4, F, 4, F, nullptr, Ff, 0.f, Fw, nullptr, nullptr), UN, "gate grid");
  expect(tg_gate_score(TG_BF16, 0, 64, 64, nullptr, 64, nullptr, nullptr, nullptr, 0.f, nullptr, nullptr, nullptr),
         TG_OK, "gate empty");
  // select
  expect(tg_select_topk(Ff, 100, 10, 11, Fo, nullptr), IA, "select q > k");
  expect(tg_select_topk(nullptr, 100, 10, 1, Fo, nullptr), IA, "select null");
  expect(tg_select_topk(Ff, 0, 10, 0, Fo, nullptr), TG_OK, "select empty");
  expect(tg_select_topk_varlen(Ff, Fi, Fi, 1 << 22, 1, 1, Fo, Fo, nullptr), UN, "select varlen grid");
  expect(tg_select_topk_varlen(Ff, nullptr, Fi, 2, 10, 1, Fo, Fo, nullptr), IA, "select varlen null");
  const int64_t ws = tg_select_topk_workspace_size(32768);
  expect(ws > 0 ? 0 : 1, 0, "select ws size");
  expect((int)tg_select_topk_workspace_size(-5), -1, "select ws size of a negative n");
  expect(tg_select_topk_ws(Ff, 32768, 4096, 64, Fo, F, ws - 4, nullptr), WS, "select ws small");
  expect(tg_select_topk_ws(Ff, 32768, 4096, 64, Fo, M, ws, nullptr), IA, "select ws align");
  // gather
  expect(tg_gather(TG_BF16, 100, 10, 8, Fi, F, 4, nullptr, F, nullptr, nullptr, nullptr), IA, "gather ld");
  expect(tg_gather(TG_BF16, 100, 10, 8, Fi, F, 8, Ff, F, nullptr, nullptr, nullptr), IA, "gather g pair");
  expect(tg_gather(TG_BF16, 1 << 27, 1 << 26, 8, Fi, F, 8, nullptr, F, nullptr, nullptr, nullptr), UN, "gather grid");
  expect(tg_gather_varlen(TG_BF16, Fi, Fi, 70000, 10, 8, Fi, F, 8, nullptr, F, nullptr, nullptr, nullptr), UN,
         "gather varlen batch");
  // rope
  expect(tg_rope_table(Fw, 100, 7, 1e4, nullptr), IA, "rope table dh");
  expect(tg_rope_table(Fw, 100, 64, 0.5, nullptr), IA, "rope table base");
  expect(tg_rope_kv(TG_BF16, 10, 4, 2, 24, Fi, Ff, 100, F, F, F, F, F, nullptr), UN, "rope dh");
  expect(tg_rope_kv(TG_BF16, 1 << 24, 1, 1, 16, Fi, Ff, 1, F, F, F, F, F, nullptr), UN, "rope grid");
  expect(tg_rope_kv(TG_BF16, 10, 4, 2, 64, Fi, Ff, 100, M, F, F, F, F, nullptr), IA, "rope align");
  // attention
  expect(tg_gated_attn(TG_BF16, 16, 6, 4, 128, 0.1f, F, F, F, nullptr, Fi, F, nullptr, nullptr), IA, "attn heads");
  expect(tg_gated_attn(TG_BF16, 16, 16, 8, 96, 0.1f, F, F, F, nullptr, Fi, F, nullptr, nullptr), UN, "attn dh");
  expect(tg_gated_attn(TG_BF16, 16, 16, 8, 128, -1.f, F, F, F, nullptr, Fi, F, nullptr, nullptr), IA, "attn scale");
  expect(tg_gated_attn(TG_FP32, 16, 70000, 70000, 64, 0.1f, F, F, F, nullptr, Fi, F, nullptr, nullptr), UN,
         "attn grid");
  expect(tg_gated_attn_varlen(TG_BF16, Fi, 70000, 16, 16, 16, 8, 128, 0.1f, F, F, F, nullptr, Fi, F, nullptr,
                              nullptr),
         UN, "attn varlen batch");
  expect(tg_gated_attn_ex(TG_BF16, nullptr, 1, 16, -1, 16, 8, 128, 0.1f, F, F, F, nullptr, nullptr, Fi, F, nullptr,
                          nullptr),
         IA, "attn ex total");
  // decode
  const int64_t dws = tg_decode_attn_workspace_size(4, 5000, 16, 8, 128);
  expect(dws > 0 ? 0 : 1, 0, "decode ws size");
  expect(tg_decode_attn(TG_BF16, Fi, 4, 5000, 16, 8, 128, 0.1f, F, F, F, nullptr, nullptr, F, nullptr, F, dws - 1,
                        nullptr),
         WS, "decode ws small");
  expect(tg_decode_attn(TG_BF16, Fi, 4, 5000, 48, 8, 128, 0.1f, F, F, F, nullptr, nullptr, F, nullptr, F, 1 << 30,
                        nullptr),
         UN, "decode group");
  // dense
  expect(tg_linear(TG_BF16, 64, 255, 64, F, 64, F, 64, nullptr, 0, F, 256, nullptr), UN, "linear n");
  expect(tg_linear(TG_FP32, 64, 256, 64, F, 64, F, 64, nullptr, 0, F, 256, nullptr), UN, "linear dtype");
  expect(tg_linear(TG_BF16, 64, 256, 64, F, 64, F, 64, F, 512, F, 256, nullptr), IA, "linear in-place ld");
  expect(tg_swiglu(TG_BF16, 64, 128, 64, F, 64, F, nullptr, 64, F, 128, nullptr), IA, "swiglu null up");
  expect(tg_qkv_proj(TG_BF16, 64, 3, 1, 128, 64, F, 64, F, 64, F, F, F, nullptr), UN, "qkv heads");
  // positions check
  expect(tg_check_positions(Fi, 10, nullptr, 0, nullptr, nullptr), IA, "check positions null");
  // status strings
  if (std::strcmp(tg_status_string(TG_OK), "TG_OK") != 0 || std::strcmp(tg_status_string(99), "TG_UNKNOWN_STATUS") != 0) {
    std::printf("MISMATCH status strings\n");
    ++g_bad;
  }
  std::printf("abi asan driver: %d mismatches\n", g_bad);
  return g_bad;
}
