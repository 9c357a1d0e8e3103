// A plain HBM read stream: the practical read ceiling the products and the attention are
// compared with (the same bytes read once with wide non-temporal loads and no arithmetic).
// Test and measurement export only; nothing on the decode path calls it.
#include "kd_internal.h"

namespace kd {

constexpr int kStreamThreads = 256;
constexpr int kStreamLoads = 4;  // 16-byte loads per lane, all in flight at once

// Workgroup w reads the 16-byte words [w * 1024, (w + 1) * 1024) of the buffer, lane l the
// words w * 1024 + l + 256 i (coalesced: 4 KB per wave-load); the words are XOR-folded and
// stored only when the fold equals a fixed constant, which keeps the loads without a store.
__global__ __launch_bounds__(kStreamThreads) void read_stream_kernel(const v4i* __restrict__ p, size_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const size_t base = (size_t)blockIdx.x * (kStreamThreads * kStreamLoads) + threadIdx.x;
  v4i v[kStreamLoads];
#pragma unroll
  for (int i = 0; i < kStreamLoads; ++i) {
    const size_t idx = base + (size_t)kStreamThreads * i;
    const v4i zero = {0, 0, 0, 0};
    v[i] = idx < n16 ? __builtin_nontemporal_load(p + idx) : zero;
  }
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < kStreamLoads; ++i) acc ^= (uint32_t)(v[i].x ^ v[i].y ^ v[i].z ^ v[i].w);
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace kd

using namespace kd;

extern "C" kd_status kd_debug_read_stream(const void* p, size_t bytes, uint32_t* sink, void* stream) {
  const char* who = "kd_debug_read_stream";
  KD_REQUIRE(p && sink, KD_ERR_INVALID, "%s: null pointer", who);
  KD_REQUIRE(bytes > 0 && bytes % 16 == 0 && aligned16(p), KD_ERR_INVALID,
             "%s: bytes=%zu must be a positive multiple of 16 and p 16-byte aligned", who, bytes);
  const size_t n16 = bytes / 16;
  const size_t per = (size_t)kStreamThreads * kStreamLoads;
  const size_t grid = (n16 + per - 1) / per;
  KD_REQUIRE(grid <= 0x7FFFFFFF, KD_ERR_UNSUPPORTED, "%s: %zu bytes is too many", who, bytes);
  read_stream_kernel<<<(unsigned)grid, kStreamThreads, 0, as_stream(stream)>>>(static_cast<const v4i*>(p), n16, sink);
  return check_launch(who);
}
