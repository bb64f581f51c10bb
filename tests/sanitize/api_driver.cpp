// Driver for the address / undefined-behaviour sanitizer build of the
// library's host code (test infrastructure): the C entry points' argument
// validation and the launch plans, run on the CPU without a GPU.  The library
// sources are compiled host-only with the sanitizers; no kernel is ever
// launched, because every call here either fails validation or, with valid
// arguments, stops at the device check.
//   * every entry point with invalid arguments returns the documented status;
//   * with valid arguments and no GPU, FP8L_ERR_DEVICE;
//   * the split-K plans over a sweep of shapes: splits cover K exactly, at most
//     one split workgroup per compute unit, partials within the fixed array of
//     fp8_block_gemm_noalloc (32 MiB) on a 256-CU device.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "../../include/fp8lin.h"
#include "../../sparse_gemm_linears_amd/csrc/launch.hpp"

static int g_bad = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      g_bad = 1;                                                            \
    }                                                                       \
  } while (0)

// fake, 16-byte aligned, non-overlapping addresses: validation fails (or the
// device check stops the call) before anything dereferences them
template <class T>
static T *fake(uintptr_t i, uintptr_t off = 0) {
  return reinterpret_cast<T *>((i << 32) + off);
}

static void validation() {
  const auto u8 = [](int i, int off = 0) { return fake<uint8_t>(i, off); };
  const auto f32 = [](int i, int off = 0) { return fake<float>(i, off); };
  const auto b16 = [](int i, int off = 0) { return fake<uint16_t>(i, off); };
  // shapes
  EXPECT(fp8_quant_act(b16(1), 4, 100, u8(2), f32(3), nullptr) == FP8L_ERR_SHAPE);
  EXPECT(fp8_quant_act(b16(1), -1, 128, u8(2), f32(3), nullptr) == FP8L_ERR_SHAPE);
  EXPECT(fp8_quant_act(b16(1), int64_t(1) << 40, 128, u8(2), f32(3), nullptr) == FP8L_ERR_SHAPE);
  EXPECT(fp8_quant_act(b16(1), int64_t(1) << 24, int64_t(1) << 24, u8(2), f32(3), nullptr) == FP8L_ERR_SHAPE);
  EXPECT(fp8_block_gemm(u8(1), f32(2), u8(3), f32(4), int64_t(1) << 24, int64_t(1) << 24, 128, fake<uint16_t>(5),
                        nullptr) == FP8L_ERR_SHAPE);
  EXPECT(fp8_grouped_gemm(u8(1), f32(2), u8(3), f32(4), fake<int32_t>(5), 4097, 16, 128, 128, b16(6), nullptr) ==
         FP8L_ERR_SHAPE);
  EXPECT(fp8_grouped_gemm(u8(1), f32(2), u8(3), f32(4), fake<int32_t>(5), 4096, 16, int64_t(1) << 24,
                          int64_t(1) << 24, b16(6), nullptr) == FP8L_ERR_SHAPE);
  EXPECT(fp8_block_gemm_swiglu(u8(1), f32(2), u8(3), f32(4), 16, 64, 128, b16(5), nullptr, nullptr, nullptr) ==
         FP8L_ERR_SHAPE);
  EXPECT(fp8_block_linear(b16(1), u8(2), f32(3), 65, 128, 128, b16(4), nullptr) == FP8L_ERR_SHAPE);
  // empty batches: OK without touching pointers
  EXPECT(fp8_quant_act(nullptr, 0, 128, nullptr, nullptr, nullptr) == FP8L_OK);
  EXPECT(fp8_block_gemm(nullptr, nullptr, u8(3), f32(4), 0, 128, 128, nullptr, nullptr) == FP8L_OK);
  EXPECT(fp8_block_gemm_noalloc(nullptr, nullptr, u8(3), f32(4), 0, 128, 128, nullptr, nullptr) == FP8L_OK);
  EXPECT(fp8_sparse24_linear(nullptr, u8(2), u8(3), f32(4), 0, 128, 128, nullptr, nullptr) == FP8L_OK);
  // null, alignment, aliasing
  EXPECT(fp8_block_gemm(u8(1), f32(2), u8(3), nullptr, 16, 128, 128, b16(5), nullptr) == FP8L_ERR_NULL);
  EXPECT(fp8_block_gemm_noalloc(u8(1), nullptr, u8(3), f32(4), 16, 128, 128, b16(5), nullptr) == FP8L_ERR_NULL);
  EXPECT(fp8_block_gemm_swiglu(u8(1), f32(2), u8(3), f32(4), 16, 128, 128, b16(5), u8(6), nullptr, nullptr) ==
         FP8L_ERR_NULL);
  EXPECT(fp8_block_gemm(u8(1), f32(2), u8(3), f32(4), 16, 128, 128, b16(5, 2), nullptr) == FP8L_ERR_ALIGN);
  EXPECT(fp8_sparse24_gemm(u8(1), f32(2), u8(3), u8(4, 1), f32(5), 16, 128, 128, b16(6), nullptr) ==
         FP8L_ERR_ALIGN);
  EXPECT(fp8_quant_act_static(b16(1), f32(2, 2), 4, 128, u8(3), f32(4), nullptr) == FP8L_ERR_ALIGN);
  EXPECT(fp8_block_gemm(u8(1), f32(2), u8(3), f32(4), 16, 128, 128, fake<uint16_t>(3, 16), nullptr) ==
         FP8L_ERR_ALIAS);
  EXPECT(fp8_block_gemm_noalloc(u8(1), f32(2), u8(3), f32(4), 16, 128, 128, fake<uint16_t>(1, 1024), nullptr) ==
         FP8L_ERR_ALIAS);
  EXPECT(prune24_compress(b16(1), nullptr, 128, 128, u8(2), u8(2, 4096), f32(3), nullptr) == FP8L_ERR_ALIAS);
  EXPECT(fp8_block_gemm_swiglu(u8(1), f32(2), u8(3), f32(4), 16, 128, 128, b16(5), u8(5, 16), f32(6), nullptr) ==
         FP8L_ERR_ALIAS);
  // status strings
  for (int s = 0; s <= 8; s++) EXPECT(fp8lin_status_str(s) != nullptr);
  EXPECT(fp8lin_status_str(1000) != nullptr);
}

static void no_device() {
  int n = 0;
  if (hipGetDeviceCount(&n) == hipSuccess && n > 0) return;  // only meaningful without a GPU
  (void)hipGetLastError();
  EXPECT(fp8_quant_act(fake<uint16_t>(1), 4, 128, fake<uint8_t>(2), fake<float>(3), nullptr) == FP8L_ERR_DEVICE);
  EXPECT(fp8_block_gemm(fake<uint8_t>(1), fake<float>(2), fake<uint8_t>(3), fake<float>(4), 128, 4096, 14336,
                        fake<uint16_t>(5), nullptr) == FP8L_ERR_DEVICE);
  EXPECT(fp8_block_gemm_noalloc(fake<uint8_t>(1), fake<float>(2), fake<uint8_t>(3), fake<float>(4), 128, 4096, 14336,
                                fake<uint16_t>(5), nullptr) == FP8L_ERR_DEVICE);
  EXPECT(fp8_sparse24_linear(fake<uint16_t>(1), fake<uint8_t>(2), fake<uint8_t>(3), fake<float>(4), 16, 4096, 14336,
                             fake<uint16_t>(5), nullptr) == FP8L_ERR_DEVICE);
  EXPECT(fp8lin_release_graph_scratch() == FP8L_OK);
}

static void plans() {
  const int cus = 256;
  const size_t fixed = size_t(32) << 20;
  size_t worst = 0;
  long checked = 0;
  for (int64_t M = 1; M <= 1200; M += (M < 80 ? 1 : 7)) {
    for (int64_t N = 128; N <= 32768; N += (N < 2048 ? 128 : 1664)) {
      for (int64_t K = 128; K <= 20480; K += (K < 2048 ? 128 : 1408)) {
        checked++;
        const size_t bytes = fp8lin::gemm_partial_bytes(M, N, K, cus);
        worst = bytes > worst ? bytes : worst;
        EXPECT(bytes <= fixed);
        if (fp8lin::use_tile_kernel(M, N, K)) {
          const fp8lin::TilePlan p = fp8lin::plan_tiles((int)M, (int)N, (int)K, cus);
          const int64_t kb = K / 128, tiles = ((M + p.bm - 1) / p.bm) * ((N + 255) / 256);
          EXPECT(p.bm == 128 || p.bm == 256);
          EXPECT(p.splits >= 1 && p.splits <= 16);
          if (p.splits > 1) {
            EXPECT(p.bm == 128);
            EXPECT(tiles * p.splits <= cus);
            EXPECT((int64_t)p.kb_split * (p.splits - 1) < kb && kb <= (int64_t)p.kb_split * p.splits);
            if (kb % 4 == 0) EXPECT(p.kb_split % 4 == 0);
            EXPECT(bytes == (size_t)p.splits * M * N * 4);
          } else {
            EXPECT(bytes == 0);
          }
        } else {
          const int s = fp8lin::decode_splits(M, N, K);
          EXPECT(M <= 64);
          EXPECT(s == 1 || s == 2 || s == 4);
          EXPECT(bytes == (s > 1 ? (size_t)s * M * N * 4 : 0));
          if (M <= 2) EXPECT(s == 1);
        }
        const size_t sw = fp8lin::swiglu_partial_bytes(M, N, K, cus);
        EXPECT(sw == 0 || sw % ((size_t)M * 2 * N * 4) == 0);
        if (M <= 64) {
          for (bool sparse : {false, true}) {
            const size_t tb = fp8lin::linear_token_bytes(M, N, K, sparse);
            // no scratch tokens exactly where the call quantizes in the kernel
            EXPECT((tb == 0) == fp8lin::linear_staged(M, N, K, sparse));
            EXPECT(tb == 0 || tb >= (size_t)M * K + (size_t)M * (K / 128) * 4);
            if (fp8lin::linear_staged(M, N, K, sparse)) EXPECT(M <= 2);
          }
        }
      }
    }
  }
  EXPECT(worst > fixed / 2);  // the array is not oversized
  std::printf("plans checked: %ld shapes, largest partials %zu bytes\n", checked, worst);
}

int main() {
  validation();
  no_device();
  plans();
  if (!g_bad) std::printf("library host sanitizer driver: ok\n");
  return g_bad;
}
