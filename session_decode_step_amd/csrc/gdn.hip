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

void launch_gdn_step(const float* q, const float* k, const float* v, const float* g, const float* beta, int B, int H,
                     const float* const* state_in, float* const* state_out, float scale, float* o, hipStream_t st) {
  RowStates rs = {};
  for (int b = 0; b < B; ++b) {
    rs.in[b] = state_in[b];
    rs.out[b] = state_out[b];
  }
  gdn_step_kernel<<<dim3(H, B), 256, 0, st>>>(q, k, v, g, beta, H, rs, scale, o);
}

// ---------------------------------------------------------------------------------------
// The pieces of a linear-attention layer around the state step (memra-engine decode_batch.rs,
// the Linear mixer of ``decode_batch_layers``: the fused conv ring, the prep, the gated norm).
// ---------------------------------------------------------------------------------------
struct ConvRows {
  const float* in[KD_MAX_B];  // the ring the step reads: [d_conv - 1][C], oldest first
  float* out[KD_MAX_B];       // the ring it writes (the row's other buffer)
};

// Sum of one value per thread over a workgroup of two waves, the same in every thread: each
// wave's lanes by row_sum, then wave 0's sum plus wave 1's (a fixed order).
__device__ __forceinline__ float sum128(float x, float* lds) {
  const float w = row_sum(x);
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = w;
  __syncthreads();
  const float t = lds[0] + lds[1];
  __syncthreads();
  return t;
}

// grid (n_v, B), 128 threads (d_state): thread i of value head h takes element i of the
// head's q and k channels (its key head kh = h / (n_v / n_k)) and of its v channel.  Each
// channel: silu of the conv over the window (the ring's d_conv - 1 inputs, then this step's),
// and the ring shifted into the row's other buffer (the q and k channels of a key head by its
// first value head only).  Then q and k L2-normalised over the head, beta = sigmoid(beta_raw),
// g = a softplus(alpha + dt).  proj rows: conv channels C = 2 d n_k + d n_v, then z (d n_v),
// then beta_raw (n_v), then alpha (n_v); row stride ldp.
__global__ __launch_bounds__(kGdnDim) void ssm_conv_prep_kernel(
    const float* __restrict__ proj, int ldp, const float* __restrict__ w, int dconv, ConvRows cr,
    const float* __restrict__ dt, const float* __restrict__ a, int nk, int nv, float eps, float* __restrict__ qo,
    float* __restrict__ ko, float* __restrict__ vo, float* __restrict__ go, float* __restrict__ bo) {
  __shared__ float lds[2];
  const int h = blockIdx.x, b = blockIdx.y, i = threadIdx.x;
  const int kh = h / (nv / nk), key_dim = kGdnDim * nk, C = 2 * key_dim + kGdnDim * nv;
  const float* x = proj + (size_t)b * ldp;
  const float* rin = cr.in[b];
  float* rout = cr.out[b];
  const int ch[3] = {kh * kGdnDim + i, key_dim + kh * kGdnDim + i, 2 * key_dim + h * kGdnDim + i};
  const bool writes_qk = (h % (nv / nk)) == 0;
  float y[3];
#pragma unroll
  for (int c3 = 0; c3 < 3; ++c3) {
    const int c = ch[c3];
    const float xn = x[c];
    float acc = 0.0f;
    for (int j = 0; j + 1 < dconv; ++j) acc = fmaf(w[(size_t)c * dconv + j], rin[(size_t)j * C + c], acc);
    acc = fmaf(w[(size_t)c * dconv + dconv - 1], xn, acc);
    y[c3] = acc / (1.0f + expf(-acc));
    if (c3 == 2 || writes_qk) {
      for (int j = 0; j + 2 < dconv; ++j) rout[(size_t)j * C + c] = rin[(size_t)(j + 1) * C + c];
      rout[(size_t)(dconv - 2) * C + c] = xn;
    }
  }
  const float sq = sum128(y[0] * y[0], lds);
  const float sk = sum128(y[1] * y[1], lds);
  const size_t o = ((size_t)b * nv + h) * kGdnDim + i;
  qo[o] = y[0] * (1.0f / sqrtf(sq + eps));
  ko[o] = y[1] * (1.0f / sqrtf(sk + eps));
  vo[o] = y[2];
  if (i == 0) {
    const float br = x[C + kGdnDim * nv + h], al = x[C + kGdnDim * nv + nv + h];
    const float t = al + dt[h];
    const float sp = t > 20.0f ? t : log1pf(expf(t));
    go[(size_t)b * nv + h] = a[h] * sp;
    bo[(size_t)b * nv + h] = 1.0f / (1.0f + expf(-br));
  }
}

void launch_ssm_conv_prep(const float* proj, int ldp, const float* w, int dconv, const float* const* ring_in,
                          float* const* ring_out, const float* dt, const float* a, int B, int nk, int nv, float eps,
                          float* q, float* k, float* v, float* g, float* beta, hipStream_t st) {
  ConvRows cr = {};
  for (int b = 0; b < B; ++b) {
    cr.in[b] = ring_in[b];
    cr.out[b] = ring_out[b];
  }
  ssm_conv_prep_kernel<<<dim3(nv, B), kGdnDim, 0, st>>>(proj, ldp, w, dconv, cr, dt, a, nk, nv, eps, q, k, v, g, beta);
}

// grid (n_v, B), 32 threads: lane l of value head h holds elements 4l .. 4l+3 of the head's
// state-step output o; y = (o / sqrt(mean(o^2) + eps)) w silu(z), quantised in blocks of 32 (8
// lanes per block) into the activation rows of the out product (k = d_state n_v).
__global__ __launch_bounds__(32) void gated_norm_quant_kernel(const float* __restrict__ o, const float* __restrict__ z,
                                                              int ldz, const float* __restrict__ wn, int nv, float eps,
                                                              int8_t* __restrict__ qs, float* __restrict__ qd) {
  const int h = blockIdx.x, b = blockIdx.y, l = threadIdx.x;
  const float4 ov = *reinterpret_cast<const float4*>(o + ((size_t)b * nv + h) * kGdnDim + 4 * l);
  const float* zr = z + (size_t)b * ldz + (size_t)h * kGdnDim + 4 * l;  // ldz need not keep 16-byte alignment
  const float4 zv = make_float4(zr[0], zr[1], zr[2], zr[3]);
  const float4 gw = *reinterpret_cast<const float4*>(wn + 4 * l);
  float ss = ov.x * ov.x;
  ss = fmaf(ov.y, ov.y, ss);
  ss = fmaf(ov.z, ov.z, ss);
  ss = fmaf(ov.w, ov.w, ss);
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 32);
  const float inv = 1.0f / sqrtf(ss / (float)kGdnDim + eps);
  const auto gate = [](float zz) { return zz / (1.0f + expf(-zz)); };
  const float4 y = make_float4(ov.x * inv * gw.x * gate(zv.x), ov.y * inv * gw.y * gate(zv.y),
                               ov.z * inv * gw.z * gate(zv.z), ov.w * inv * gw.w * gate(zv.w));
  const int NQ = n_quads(kGdnDim * nv), nbp = NQ * 4;
  const int blk = h * (kGdnDim / 32) + l / 8;
  quant4_lane8(y, l & 7, true, qs + ((size_t)b * NQ + (blk >> 2)) * 128 + (blk & 3) * 8, qd + (size_t)b * nbp + blk);
}

void launch_gated_norm_quant(const float* o, const float* z, int ldz, const float* w, int B, int nv, float eps,
                             int8_t* qs, float* qd, hipStream_t st) {
  gated_norm_quant_kernel<<<dim3(nv, B), 32, 0, st>>>(o, z, ldz, w, nv, eps, qs, qd);
}

int gdn_state_dim() { return kGdnDim; }

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
