// Greedy next token of each row, the embedding gather that turns tokens into the next
// step's input rows, and the accepted prefix of speculative-verify rows.
//
// What is computed (memra-engine 0.72.0, src/decode_batch.rs): ``decode_step_batch_sampled``
// picks, for each greedy row, the device argmax of its logits row between the lm_head product
// and the logits readback, and states that it equals the host argmax bit for bit; phase 0 of
// ``decode_step_batch`` starts each row from the embedding row of its token.  Reading of the
// tie rule (the pages do not state one): the lowest index among equal maxima, as a host scan
// that keeps the first maximum finds.
//
// How: one workgroup per row.  Every lane scans a strided share of the row keeping its first
// maximum; lanes, then waves, are merged with "larger value wins, equal values keep the lower
// index" -- a total order, so the result does not depend on the merge tree.  NaN entries never
// win.  No arithmetic touches the values: the result is exact.
//
// Verify rows (Strata PR #1524, "What changes": wider target verification across concurrent
// streams with accepted-prefix state commits): a stream's k rows hold, in order, its last
// committed token and k - 1 draft tokens at consecutive positions; row j's greedy token is the
// target's choice after row j's input.  Reading (greedy verification; the page does not spell
// out the rule): draft j + 1 is kept while it equals row j's greedy token, the first mismatch
// ends the prefix, and the token after the kept prefix is the greedy token of its last row.
#include <climits>

#include "kd_internal.h"

namespace kd {

constexpr int kArgmaxThreads = 1024;
constexpr int kArgmaxUnroll = 8;

// Merge candidate (v2, i2) into (v, i); i == INT_MAX marks "no entry yet".
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (i2 == INT_MAX || v2 != v2) return;
  if (i == INT_MAX || v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__global__ __launch_bounds__(kArgmaxThreads) void argmax_rows_kernel(const float* __restrict__ x, int n, int ldx,
                                                                     int32_t* __restrict__ idx,
                                                                     float* __restrict__ val) {
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const float* row = x + (size_t)b * ldx;
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int j0 = t; j0 < n; j0 += kArgmaxUnroll * kArgmaxThreads) {
    float v[kArgmaxUnroll];
#pragma unroll
    for (int u = 0; u < kArgmaxUnroll; ++u) {
      const int j = j0 + u * kArgmaxThreads;
      v[u] = j < n ? row[j] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kArgmaxUnroll; ++u) {
      const int j = j0 + u * kArgmaxThreads;
      argmax_merge(bv, bi, v[u], j < n ? j : INT_MAX);
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float v2 = __shfl_xor(bv, m, 64);
    const int i2 = __shfl_xor(bi, m, 64);
    argmax_merge(bv, bi, v2, i2);
  }
  __shared__ float sv[kArgmaxThreads / 64];
  __shared__ int si[kArgmaxThreads / 64];
  if (lane == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  if (t == 0) {
    for (int ww = 1; ww < kArgmaxThreads / 64; ++ww) argmax_merge(bv, bi, sv[ww], si[ww]);
    idx[b] = bi == INT_MAX ? 0 : bi;  // a row of NaN only: index 0
    if (val) val[b] = bi == INT_MAX ? __int_as_float(0x7FC00000) : bv;
  }
}

// grid (ceil(d / 256), B): out[b][:] = table[tokens[b]][:], or zeros for a token outside
// [0, vocab) (no read).
__global__ __launch_bounds__(256) void embed_rows_kernel(const float* __restrict__ table, int vocab, int d,
                                                         const int32_t* __restrict__ tokens, float* __restrict__ out,
                                                         int ldo) {
  const int b = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  const int tok = tokens[b];
  const bool valid = tok >= 0 && tok < vocab;
  out[(size_t)b * ldo + c] = valid ? table[(size_t)tok * d + c] : 0.0f;
}

// One thread per stream: the accepted prefix of its drafts and the token that follows it.
__global__ void verify_accept_kernel(const int32_t* __restrict__ greedy, const int32_t* __restrict__ fed,
                                     int n_streams, int k, int32_t* __restrict__ n_accept,
                                     int32_t* __restrict__ next_token) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n_streams) return;
  const int32_t* g = greedy + (size_t)s * k;
  const int32_t* f = fed + (size_t)s * k;
  int a = 0;
  while (a + 1 < k && g[a] == f[a + 1]) ++a;
  n_accept[s] = a;
  next_token[s] = g[a];
}

}  // namespace kd

using namespace kd;

extern "C" kd_status kd_verify_accept(const int32_t* greedy, const int32_t* fed, int32_t n_streams, int32_t k,
                                      int32_t* n_accept, int32_t* next_token, void* stream) {
  KD_REQUIRE(n_streams >= 1 && n_streams <= KD_MAX_B, KD_ERR_UNSUPPORTED, "kd_verify_accept: n_streams=%d outside [1,16]",
             n_streams);
  KD_REQUIRE(k >= 1 && n_streams * k <= KD_MAX_B, KD_ERR_UNSUPPORTED,
             "kd_verify_accept: %d streams x %d rows outside one step's 16 rows", n_streams, k);
  KD_REQUIRE(greedy && fed && n_accept && next_token, KD_ERR_INVALID, "kd_verify_accept: null pointer");
  verify_accept_kernel<<<1, 64, 0, as_stream(stream)>>>(greedy, fed, n_streams, k, n_accept, next_token);
  return check_launch("kd_verify_accept");
}

extern "C" kd_status kd_argmax_rows(const float* x, int32_t B, int32_t n, int32_t ldx, int32_t* idx, float* val,
                                    void* stream) {
  KD_REQUIRE(B >= 1 && B <= 65535, KD_ERR_UNSUPPORTED, "kd_argmax_rows: B=%d outside [1, 65535]", B);
  KD_REQUIRE(n >= 1, KD_ERR_INVALID, "kd_argmax_rows: n=%d < 1", n);
  KD_REQUIRE(ldx >= n, KD_ERR_INVALID, "kd_argmax_rows: ldx=%d < n=%d", ldx, n);
  KD_REQUIRE(x && idx, KD_ERR_INVALID, "kd_argmax_rows: null pointer");
  argmax_rows_kernel<<<B, kArgmaxThreads, 0, as_stream(stream)>>>(x, n, ldx, idx, val);
  return check_launch("kd_argmax_rows");
}

extern "C" kd_status kd_embed_rows(const float* table, int32_t vocab, int32_t d, const int32_t* tokens, int32_t B,
                                   float* out, int32_t ldo, void* stream) {
  KD_REQUIRE(B >= 1 && B <= 65535, KD_ERR_UNSUPPORTED, "kd_embed_rows: B=%d outside [1, 65535]", B);
  KD_REQUIRE(vocab >= 1 && d >= 1, KD_ERR_INVALID, "kd_embed_rows: vocab=%d d=%d", vocab, d);
  KD_REQUIRE(ldo >= d, KD_ERR_INVALID, "kd_embed_rows: ldo=%d < d=%d", ldo, d);
  KD_REQUIRE(table && tokens && out, KD_ERR_INVALID, "kd_embed_rows: null pointer");
  embed_rows_kernel<<<dim3(ceil_div(d, 256), B), 256, 0, as_stream(stream)>>>(table, vocab, d, tokens, out, ldo);
  return check_launch("kd_embed_rows");
}
