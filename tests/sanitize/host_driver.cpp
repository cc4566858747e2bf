// Host layer of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer,
// built with a plain C++ compiler and no GPU: the kernel launchers are replaced
// by stubs that count launches, and every entry point is driven with valid and
// invalid arguments.  An invalid call must return an error status and launch
// nothing; a valid one must launch.  Exit status 0 means every check passed.
#include <cmath>
#include <cstdio>
#include <cstdlib>

#include "../../bit_quantized_decode_dqk_amd/csrc/dqk_host.h"

static int g_launches = 0;
static int g_failures = 0;

namespace dqk {
int compute_units() { return 256; }
bool decode4_supported(const dqk_cache &c, int hq) {
  return c.capacity % 64 == 0 && hq % (c.num_kv_heads * 4) == 0;
}
hipError_t decode_scratch(float **ptr) {
  *ptr = reinterpret_cast<float *>(0x7000000);
  return hipSuccess;
}
#define STUB ++g_launches; return hipSuccess;
hipError_t launch_append(const dqk_cache &, const void *, const void *, bool, const float *,
                         const int32_t *, int, hipStream_t) { STUB }
hipError_t launch_select(const void *, bool, const float *, int, int, int, int, int, float *,
                         int32_t *, hipStream_t) { STUB }
hipError_t launch_select_shared(const void *, bool, const float *, int, int, int, int, int,
                                float *, int32_t *, hipStream_t) { STUB }
hipError_t launch_append_select(const dqk_cache &, const void *, const void *, bool, const float *,
                                const int32_t *, int, const void *, const float *, int, int,
                                float *, int32_t *, hipStream_t) { STUB }
hipError_t launch_decode(const dqk_cache &, const float *, const int32_t *, bool, int, int, float,
                         int, bool, float *, float *, hipStream_t) { STUB }
hipError_t launch_decode4(const dqk_cache &, const float *, const int32_t *, bool, int, int, float,
                          int, bool, float *, float *, hipStream_t) { STUB }
hipError_t launch_dequant(const dqk_cache &, float *, float *, hipStream_t) { STUB }
hipError_t launch_cache_grow(const dqk_cache &, const dqk_cache &, hipStream_t) { STUB }
hipError_t launch_bf16_decode(const uint16_t *, const uint16_t *, const uint16_t *, const int32_t *,
                              int, int, int, int, int, float, int, float *, float *,
                              hipStream_t) { STUB }
hipError_t launch_combine(const float *, int, int, int, int, int, float *, hipStream_t) { STUB }
hipError_t launch_f16_convert(const float *, uint16_t *, size_t, hipStream_t) { STUB }
hipError_t launch_stream_read(const void *, size_t, uint32_t *, int, int, hipStream_t) { STUB }
}  // namespace dqk

// status `got` must equal `want`; a call expected to fail must not launch
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int before = g_launches;                                                      \
    const dqk_status got = (call);                                                      \
    const bool launched = g_launches != before;                                         \
    if (got != (want) || launched != ((want) == DQK_OK && expect_launch)) {             \
      std::fprintf(stderr, "line %d: %s -> %d (want %d), launched %d\n", __LINE__,      \
                   #call, (int)got, (int)(want), (int)launched);                        \
      ++g_failures;                                                                     \
    }                                                                                   \
  } while (0)

static dqk_cache fake(int batch, int hkv, int d, int cap, uintptr_t base = 0x100000) {
  dqk_cache c;
  c.batch = batch;
  c.num_kv_heads = hkv;
  c.head_dim = d;
  c.capacity = cap;
  c.k_codes = reinterpret_cast<uint8_t *>(base);
  c.k_scales = reinterpret_cast<uint16_t *>(base + 0x1000000);
  c.k_ch0 = reinterpret_cast<uint16_t *>(base + 0x2000000);
  c.k_tail = reinterpret_cast<float *>(base + 0x3000000);
  c.v_codes = reinterpret_cast<uint32_t *>(base + 0x4000000);
  c.v_scales = reinterpret_cast<uint16_t *>(base + 0x5000000);
  c.lengths = reinterpret_cast<int32_t *>(base + 0x6000000);
  return c;
}

int main() {
  bool expect_launch = false;
  const dqk_cache c = fake(2, 2, 128, 256);
  const void *P = reinterpret_cast<void *>(0x8000000);
  float *F = reinterpret_cast<float *>(0x9000000);
  int32_t *I = reinterpret_cast<int32_t *>(0xA000000);
  uint16_t *H = reinterpret_cast<uint16_t *>(0xB000000);
  uint32_t *U = reinterpret_cast<uint32_t *>(0xC000000);
  size_t sizes[7];
  int32_t keep = 0;
  size_t ws = 0;

  // host queries
  EXPECT(dqk_keep_count(128, 40, &keep), DQK_OK);
  if (keep != 77) ++g_failures;
  EXPECT(dqk_keep_count(0, 40, &keep), DQK_ERR_INVALID);
  EXPECT(dqk_keep_count(128, 101, &keep), DQK_ERR_INVALID);
  EXPECT(dqk_keep_count(128, 40, nullptr), DQK_ERR_INVALID);
  EXPECT(dqk_cache_plane_bytes(1, 8, 128, 131104, sizes), DQK_OK);
  EXPECT(dqk_cache_plane_bytes(1, 8, 96, 131104, sizes), DQK_ERR_UNSUPPORTED);
  EXPECT(dqk_cache_plane_bytes(1, 8, 128, 100, sizes), DQK_ERR_INVALID);
  EXPECT(dqk_decode_workspace_bytes(&c, 8, 0, &ws), DQK_OK);
  EXPECT(dqk_decode_workspace_bytes(&c, 8, 48, &ws), DQK_ERR_INVALID);
  EXPECT(dqk_decode_workspace_bytes(nullptr, 8, 0, &ws), DQK_ERR_INVALID);
  EXPECT(dqk_bf16_decode_workspace_bytes(1, 32, 8, 128, 131072, 0, &ws), DQK_OK);
  for (int s = -4; s < 4; ++s) std::printf("%s\n", dqk_status_str(static_cast<dqk_status>(s)));

  // invalid calls: an error status and no launch
  EXPECT(dqk_transform_quantize_append(&c, nullptr, P, DQK_BF16, F, I, 4, nullptr), DQK_ERR_INVALID);
  EXPECT(dqk_transform_quantize_append(&c, P, P, DQK_BF16, F, I, 257, nullptr), DQK_ERR_INVALID);
  EXPECT(dqk_select_channels(P, DQK_BF16, F, 2, 8, 2, 128, 0, F, I, nullptr), DQK_ERR_INVALID);
  EXPECT(dqk_select_channels(P, DQK_BF16, F, 2, 6, 2, 128, 77, F, I, nullptr), DQK_ERR_UNSUPPORTED);
  EXPECT(dqk_select_channels_shared(P, DQK_BF16, F, 2, 8, 2, 128, 129, F, I, nullptr), DQK_ERR_INVALID);
  EXPECT(dqk_append_select(&c, P, P, F, I, 1, P, F, 7, 77, DQK_BF16, F, I, nullptr), DQK_ERR_INVALID);
  EXPECT(dqk_decode_attention(&c, F, I, 8, 77, NAN, 0, F, U, 1 << 30, nullptr), DQK_ERR_INVALID);
  EXPECT(dqk_decode_attention(&c, F, I, 8, 77, 0.1f, 0, F, nullptr, 1 << 30, nullptr), DQK_ERR_WORKSPACE);
  EXPECT(dqk_decode_attention_shared(&c, F, I, 8, 0, 0.1f, 0, F, U, 1 << 30, nullptr), DQK_ERR_INVALID);
  const dqk_cache big = fake(64, 8, 128, 131072);
  EXPECT(dqk_decode_attention_noalloc(&big, F, I, 32, 77, 0.1f, 256, F, nullptr), DQK_ERR_WORKSPACE);
  const dqk_cache grown = fake(2, 2, 128, 512, 0x20000000);
  EXPECT(dqk_cache_grow(&c, &c, nullptr), DQK_ERR_INVALID);
  EXPECT(dqk_cache_grow(&grown, &c, nullptr), DQK_ERR_INVALID);
  EXPECT(dqk_dequant_reference(&c, nullptr, F, nullptr), DQK_ERR_INVALID);
  EXPECT(dqk_bf16_decode_attention(H, H, H, I, 1, 24, 8, 128, 1024, 0.1f, 0, F, U, 1 << 30, nullptr),
         DQK_ERR_UNSUPPORTED);
  EXPECT(dqk_debug_f16_from_f32(nullptr, H, 4, nullptr), DQK_ERR_INVALID);
  EXPECT(dqk_stream_read(P, 24, U, nullptr), DQK_ERR_INVALID);
  EXPECT(dqk_stream_read_config(P, 1 << 20, U, 0, 4, nullptr), DQK_ERR_INVALID);

  // valid calls: OK and a launch
  expect_launch = true;
  EXPECT(dqk_transform_quantize_append(&c, P, P, DQK_BF16, F, I, 4, nullptr), DQK_OK);
  EXPECT(dqk_select_channels(P, DQK_F32, F, 2, 8, 2, 128, 77, F, I, nullptr), DQK_OK);
  EXPECT(dqk_select_channels_shared(P, DQK_BF16, F, 2, 8, 2, 128, 77, F, I, nullptr), DQK_OK);
  EXPECT(dqk_append_select(&c, P, P, F, I, 1, P, F, 8, 77, DQK_BF16, F, I, nullptr), DQK_OK);
  EXPECT(dqk_decode_attention(&c, F, I, 8, 77, 0.1f, 0, F, U, 1 << 30, nullptr), DQK_OK);
  EXPECT(dqk_decode_attention_shared(&c, F, I, 8, 77, 0.1f, 64, F, U, 1 << 30, nullptr), DQK_OK);
  EXPECT(dqk_decode_attention_noalloc(&c, F, I, 8, 77, 0.1f, 0, F, nullptr), DQK_OK);
  EXPECT(dqk_cache_grow(&c, &grown, nullptr), DQK_OK);
  EXPECT(dqk_dequant_reference(&c, F, F, nullptr), DQK_OK);
  EXPECT(dqk_bf16_decode_attention(H, H, H, I, 1, 32, 8, 128, 1024, 0.1f, 0, F, U, 1 << 30, nullptr),
         DQK_OK);
  EXPECT(dqk_debug_f16_from_f32(F, H, 4, nullptr), DQK_OK);
  EXPECT(dqk_stream_read(P, 1 << 20, U, nullptr), DQK_OK);
  EXPECT(dqk_stream_read_config(P, 1 << 20, U, 512, 8, nullptr), DQK_OK);

  // the default split rule over many shapes (integer arithmetic, no overflow)
  expect_launch = false;
  for (int batch : {1, 3, 16, 64})
    for (int hkv : {1, 2, 8})
      for (int cap : {32, 64, 96, 4096, 65536, 131072, 1 << 20})
        for (int g : {1, 2, 4, 8}) {
          const dqk_cache x = fake(batch, hkv, 128, cap);
          EXPECT(dqk_decode_workspace_bytes(&x, g * hkv, 0, &ws), DQK_OK);
        }

  // The matrix-core decode's uneven shares (the function the kernel runs), over
  // the first-slot counts the library produces (fs >= nsplit / 2, fs < nsplit):
  // the splits partition the row in order, no split needs more chunks than an
  // even share, and the 32-bit products stay in range.
  {
    auto chunks = [](int n) { return n <= 1 ? 1 : (n - 2) / dqk::kDecodeChunkBlocks + 1; };
    long applied = 0, bad = 0;
    for (int nsplit : {2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 128, 255, 256, 511,
                       512, 1000, 2047, 4096, 8191})
      for (int fs : {nsplit / 2, nsplit / 2 + 1, (3 * nsplit) / 4, nsplit - 1}) {
        if (fs < nsplit / 2 || fs >= nsplit) continue;
        const int step = nsplit < 64 ? 1 : nsplit / 32;
        for (int nblk = 1; nblk <= 52 * nsplit; nblk += step)
          for (int cut = 0; cut < 2; ++cut) {
            const dqk::SplitShares sh = dqk::uneven_shares(nblk, nsplit, fs, cut);
            if (sh.second < 0) continue;
            ++applied;
            const int even = (nblk + nsplit - 1) / nsplit;
            bool ok = (unsigned long long)sh.first_total * (unsigned long long)fs < (1ull << 32) &&
                      sh.first_total >= 0;
            int pos = 0;
            for (int s = 0; s < nsplit && ok; ++s) {
              const dqk::BlockRange r = dqk::uneven_split_range(sh, s, fs, nsplit, nblk);
              ok = r.lo == pos && r.hi >= r.lo && chunks(r.hi - r.lo) <= chunks(even);
              pos = r.hi;
            }
            if (!ok || pos != nblk) {
              if (++bad <= 5)
                std::fprintf(stderr, "uneven shares: nblk %d nsplit %d fs %d cut %d\n", nblk, nsplit, fs, cut);
            }
          }
      }
    std::printf("uneven shares: %ld cases, %ld bad\n", applied, bad);
    if (bad != 0 || applied == 0) ++g_failures;
  }
  std::printf("launches %d, failures %d\n", g_launches, g_failures);
  return g_failures == 0 ? 0 : 1;
}
