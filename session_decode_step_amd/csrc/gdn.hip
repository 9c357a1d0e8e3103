// One decode step of the gated delta rule over B rows' recurrent states (linear-attention
// layers).
//
// What is computed (memra-engine 0.72.0, src/decode_batch.rs, the Linear mixer of
// ``decode_batch_layers``: after the batched projections and the prep launch, one batched
// scan launch reads each sequence's state through the per-row pointer table and writes its
// other buffer, with scale 1/sqrt(d_state) and d_state = 128; the update is the published
// gated delta rule): per row b and value head h, with state S [d_v][d_k] fp32,
//   S' = exp(g) S,   u = S' k,   S_new = S' + beta (v - u) k^T,   o = scale S_new q.
//
// How: one workgroup of 4 waves per (head, row).  Wave w owns state rows v = 32w .. 32w+31
// and lane l the columns 2l, 2l+1 of each, so every row is one coalesced 512-byte access.
// All 32 rows are loaded before the first is used; u and o of each row are sums over the 64
// lanes in a fixed order (row_sum), so a row's result does not depend on B.  Each lane writes back only the elements it read: the step may run
// in place (state_in == state_out).
#include "kd_internal.h"

namespace kd {

constexpr int kGdnDim = 128;  // d_state: d_k = d_v = 128
constexpr int kGdnRowsPerWave = 32;

// Sum over the 64 lanes, the same value in every lane, without LDS: DPP adds within each
// 16-lane row (partner lanes l^1, l^2, then the mirrored lane of the half row and of the row),
// then the four row sums read from lanes 0, 16, 32, 48 and added in that order.
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp_f<0x141>(x);  // row_half_mirror: lane 7 - i of the half row (the other quad)
  x += dpp_f<0x140>(x);  // row_mirror: lane 15 - i of the row (the other half row)
  return ((lane_f(x, 0) + lane_f(x, 16)) + lane_f(x, 32)) + lane_f(x, 48);
}

struct RowStates {
  const float* in[KD_MAX_B];
  float* out[KD_MAX_B];
};

__global__ __launch_bounds__(256) void gdn_step_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                       const float* __restrict__ v, const float* __restrict__ g,
                                                       const float* __restrict__ beta, int H, RowStates st,
                                                       float scale, float* __restrict__ o) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t hv = (size_t)b * H + h;
  const float* Sin = st.in[b] + (size_t)h * kGdnDim * kGdnDim;
  float* Sout = st.out[b] + (size_t)h * kGdnDim * kGdnDim;
  const int v0 = w * kGdnRowsPerWave;
  float2 s[kGdnRowsPerWave];
#pragma unroll
  for (int j = 0; j < kGdnRowsPerWave; ++j)
    s[j] = *reinterpret_cast<const float2*>(Sin + (size_t)(v0 + j) * kGdnDim + 2 * lane);
  const float2 k2 = *reinterpret_cast<const float2*>(k + hv * kGdnDim + 2 * lane);
  const float2 q2 = *reinterpret_cast<const float2*>(q + hv * kGdnDim + 2 * lane);
  const float vl = lane < kGdnRowsPerWave ? v[hv * kGdnDim + v0 + lane] : 0.0f;  // lane j: v of row v0 + j
  const float a = expf(g[hv]);
  const float bt = beta[hv];
  float ol = 0.0f;  // lane j < 32 keeps o of row v0 + j
#pragma unroll
  for (int j = 0; j < kGdnRowsPerWave; ++j) {
    const float sx = a * s[j].x, sy = a * s[j].y;
    const float u = row_sum(fmaf(sx, k2.x, sy * k2.y));
    const float c = bt * (__shfl(vl, j, 64) - u);
    const float nx = fmaf(c, k2.x, sx), ny = fmaf(c, k2.y, sy);
    *reinterpret_cast<float2*>(Sout + (size_t)(v0 + j) * kGdnDim + 2 * lane) = make_float2(nx, ny);
    const float oj = row_sum(fmaf(nx, q2.x, ny * q2.y));
    if (lane == j) ol = oj;
  }
  if (lane < kGdnRowsPerWave) o[hv * kGdnDim + v0 + lane] = scale * ol;
}

}  // namespace kd

using namespace kd;

extern "C" kd_status kd_gdn_step(const float* q, const float* k, const float* v, const float* g, const float* beta,
                                 int32_t B, int32_t n_heads, int32_t d_state, const void* const* state_in,
                                 void* const* state_out, float scale, float* o, void* stream) {
  KD_REQUIRE(B >= 1 && B <= KD_MAX_B, KD_ERR_UNSUPPORTED, "kd_gdn_step: B=%d outside [1,16]", B);
  KD_REQUIRE(n_heads >= 1 && n_heads <= 65535, KD_ERR_INVALID, "kd_gdn_step: n_heads=%d", n_heads);
  KD_REQUIRE(d_state == kGdnDim, KD_ERR_UNSUPPORTED, "kd_gdn_step: d_state=%d (only 128)", d_state);
  KD_REQUIRE(q && k && v && g && beta && state_in && state_out && o, KD_ERR_INVALID, "kd_gdn_step: null pointer");
  RowStates st = {};
  for (int b = 0; b < B; ++b) {
    KD_REQUIRE(state_in[b] && state_out[b], KD_ERR_INVALID, "kd_gdn_step: null state pointer for row %d", b);
    for (int a = 0; a < b; ++a) {
      KD_REQUIRE(state_out[a] != state_out[b], KD_ERR_INVALID, "kd_gdn_step: rows %d and %d write the same state", a,
                 b);
      KD_REQUIRE(state_out[a] != state_in[b] && state_out[b] != state_in[a], KD_ERR_INVALID,
                 "kd_gdn_step: rows %d and %d: one writes the state the other reads", a, b);
    }
    st.in[b] = static_cast<const float*>(state_in[b]);
    st.out[b] = static_cast<float*>(state_out[b]);
  }
  gdn_step_kernel<<<dim3(n_heads, B), 256, 0, as_stream(stream)>>>(q, k, v, g, beta, n_heads, st, scale, o);
  return check_launch("kd_gdn_step");
}
