// host_driver.cpp -- calls every entry point of libtopk.h with arguments its
// checks reject (and with nothing to do), in a build of the library's host
// code with -fsanitize=address,undefined: each call must return the
// documented status before any GPU work, leave a reason in
// topk_last_error(), and touch no memory out of bounds.  Pointers are fake,
// non-null, and never dereferenced by the checks.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "libtopk.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  const char* why = topk_last_error();
  if (got != want || (want != 0 && (!why || !why[0]))) {
    std::printf("FAIL %s: status %d, want %d (%s)\n", what, got, want, why ? why : "null");
    ++failures;
  }
}

int main() {
  const uint16_t* L = reinterpret_cast<const uint16_t*>(uintptr_t(0x10000));
  const int32_t* VL = reinterpret_cast<const int32_t*>(uintptr_t(0x20000));
  int32_t* O = reinterpret_cast<int32_t*>(uintptr_t(0x30000));
  int32_t* V = reinterpret_cast<int32_t*>(uintptr_t(0x40000));
  int32_t* I = reinterpret_cast<int32_t*>(uintptr_t(0x50000));
  const uint16_t* TP = reinterpret_cast<const uint16_t*>(uintptr_t(0x60000));
  uint16_t* TW = reinterpret_cast<uint16_t*>(uintptr_t(0x70000));
  const int32_t* PG = reinterpret_cast<const int32_t*>(uintptr_t(0x80000));
  topk_block_table_t bt = {PG, 4, 64};
  topk_block_table_t bad_p = {PG, 4, 48};
  topk_block_table_t short_bt = {PG, 1, 64};
  topk_block_table_t null_bt = {nullptr, 4, 64};
  topk_options_t opt = {0, nullptr};

  expect("k 0", topk_bf16_rows(L, 256, VL, 4, 256, 0, 0, nullptr, O, nullptr), -1);
  expect("k 2049", topk_bf16_rows(L, 256, VL, 4, 256, 2049, 0, nullptr, O, nullptr), -1);
  expect("mode 2", topk_bf16_rows(L, 256, VL, 4, 256, 8, 2, nullptr, O, nullptr), -1);
  expect("rows -1", topk_bf16_rows(L, 256, VL, -1, 256, 8, 0, nullptr, O, nullptr), -1);
  expect("width", topk_bf16_rows(L, (1 << 20) + 8, VL, 4, (1 << 20) + 8, 8, 0, nullptr, O,
                                 nullptr), -1);
  expect("stride < width", topk_bf16_rows(L, 128, VL, 4, 256, 8, 0, nullptr, O, nullptr), -1);
  expect("stride % 8", topk_bf16_rows(L, 260, VL, 4, 256, 8, 0, nullptr, O, nullptr), -2);
  expect("null logits", topk_bf16_rows(nullptr, 256, VL, 4, 256, 8, 0, nullptr, O, nullptr), -1);
  expect("logits align", topk_bf16_rows(L + 1, 256, VL, 4, 256, 8, 0, nullptr, O, nullptr), -2);
  expect("out align", topk_bf16_rows(L, 256, VL, 4, 256, 8, 0, nullptr,
                                     reinterpret_cast<int32_t*>(uintptr_t(0x30002)), nullptr), -2);
  expect("null table pages", topk_bf16_rows(L, 256, VL, 4, 256, 8, 0, &null_bt, O, nullptr), -1);
  expect("page size", topk_bf16_rows(L, 256, VL, 4, 256, 8, 0, &bad_p, O, nullptr), -1);
  expect("table rows", topk_bf16_rows(L, 256, VL, 4, 256, 8, 0, &short_bt, O, nullptr), -1);
  expect("rows 0", topk_bf16_rows(nullptr, 256, nullptr, 0, 256, 8, 0, nullptr, nullptr, nullptr),
         0);
  expect("ex k 0", topk_bf16_rows_ex(L, 256, VL, 4, 256, 0, 0, &bt, O, &opt, nullptr), -1);
  expect("noalloc k 0", topk_bf16_rows_noalloc(L, 256, VL, 4, 256, 0, 0, nullptr, O, nullptr), -1);
  expect("noalloc align", topk_bf16_rows_noalloc(L + 4, 256, VL, 4, 256, 8, 0, nullptr, O,
                                                 nullptr), -2);
  expect("ordered valid align", topk_bf16_rows_ordered(L, 256, VL, 4, 256, 8, 0, nullptr, O,
                                                       V + 0, reinterpret_cast<int32_t*>(
                                                           uintptr_t(0x50001)), nullptr), -2);
  expect("ordered_ex mode", topk_bf16_rows_ordered_ex(L, 256, VL, 4, 256, 8, 3, nullptr, O, V, I,
                                                      &opt, nullptr), -1);
  expect("tops null", topk_bf16_rows_tops(L, 256, VL, 4, 256, 8, 0, nullptr, 32, nullptr, O,
                                          nullptr, nullptr), -1);
  expect("tops align", topk_bf16_rows_tops(L, 256, VL, 4, 256, 8, 0, TP + 1, 32, nullptr, O,
                                           nullptr, nullptr), -2);
  expect("tops stride", topk_bf16_rows_tops(L, 256, VL, 4, 256, 8, 0, TP, 24, nullptr, O,
                                            nullptr, nullptr), -1);
  expect("maxima stride", topk_bf16_vector_maxima(L, 256, VL, 4, 256, TW, 12, nullptr), -2);
  expect("maxima rows -1", topk_bf16_vector_maxima(L, 256, VL, -1, 256, TW, 32, nullptr), -1);
  expect("maxima nothing", topk_bf16_vector_maxima(nullptr, 256, nullptr, 0, 256, nullptr, 0,
                                                   nullptr), 0);
  const uint8_t* QB = reinterpret_cast<const uint8_t*>(uintptr_t(0x90000));
  const uint8_t* KB = reinterpret_cast<const uint8_t*>(uintptr_t(0xA0000));
  const uint8_t* SB = reinterpret_cast<const uint8_t*>(uintptr_t(0xB0000));
  const uint16_t* WB = reinterpret_cast<const uint16_t*>(uintptr_t(0xC0000));
  uint16_t* LB = reinterpret_cast<uint16_t*>(uintptr_t(0xD0000));
  expect("score qpr 9", topk_fp8_mqa_logits(QB, WB, KB, SB, 100, VL, 9, 9, 100, LB, 100, TW, 16,
                                            nullptr), -1);
  expect("score rows", topk_fp8_mqa_logits(QB, WB, KB, SB, 100, VL, 5, 2, 100, LB, 100, TW, 16,
                                           nullptr), -1);
  expect("score key stride", topk_fp8_mqa_logits(QB, WB, KB, SB, 99, VL, 4, 2, 100, LB, 100, TW,
                                                 16, nullptr), -1);
  expect("score q aligned", topk_fp8_mqa_logits(QB + 8, WB, KB, SB, 100, VL, 4, 2, 100, LB, 100,
                                                TW, 16, nullptr), -2);
  expect("score null", topk_fp8_mqa_logits(QB, WB, nullptr, SB, 100, VL, 4, 2, 100, LB, 100, TW,
                                           16, nullptr), -1);
  expect("score nothing", topk_fp8_mqa_logits(nullptr, nullptr, nullptr, nullptr, 0, nullptr, 0,
                                              1, 100, nullptr, 0, nullptr, 0, nullptr), 0);
  expect("mxfp4 q scale null", topk_mxfp4_mqa_logits(QB, nullptr, WB, KB, SB, 100, VL, 4, 2, 100,
                                                     LB, 100, TW, 16, nullptr), -1);
  expect("mxfp4 keys aligned", topk_mxfp4_mqa_logits(QB, SB, WB, KB + 4, SB, 100, VL, 4, 2, 100,
                                                     LB, 100, TW, 16, nullptr), -2);
  expect("mxfp4 tops stride", topk_mxfp4_mqa_logits(QB, SB, WB, KB, SB, 100, VL, 4, 2, 100, LB,
                                                    100, TW, 12, nullptr), -1);
  expect("mxfp4 nothing", topk_mxfp4_mqa_logits(nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                                                nullptr, 0, 1, 100, nullptr, 0, nullptr, 0,
                                                nullptr), 0);
  expect("reserve k", topk_reserve_scratch(4, 1 << 20, 0, 0, 0, nullptr), -1);
  expect("reserve one workgroup", topk_reserve_scratch(4, 16384, 8, 0, 1, nullptr), 0);
  for (int s = -6; s <= 1; ++s) {
    const char* name = topk_status_string(s);
    if (!name || !name[0] || std::strlen(name) > 200) {
      std::printf("FAIL status string %d\n", s);
      ++failures;
    }
  }
  std::printf("host driver: %d failure(s)\n", failures);
  return failures ? 1 : 0;
}
