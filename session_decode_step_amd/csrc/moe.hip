// Mixture-of-experts FFN for a batch of rows with experts merged across rows.
//
// What is computed (hf2q ADR-040 §0.7 F4: per-token top-k routing, rows grouped by expert so
// each active expert's weights are read once and applied to every row routed to it, then a
// per-row weighted sum; Strata pull request #1524 "What changes": merged expert execution
// and a shared expert): r = W_r z (fp32 router), the top-k experts by descending logit
// (ties to the lower id), p = softmax over the k selected logits, moe_b = sum_k p_k
// Expert_{e_k}(z_b) in rank order, plus the shared expert's output.
//
// How: routing and grouping run on the device (no host round trip).  The routing kernel
// also lists, for each expert, the (row, rank) pairs routed to it in ascending row order; the
// grouped mmvq reads each active expert's tiles once (empty experts exit before reading)
// and treats its rows as the MFMA's activation rows, whose results never depend on which
// other rows share the expert; the shared expert's down product adds the k expert outputs of
// a row in rank order to its own (its epilogue).  So a row's result is the same at any B.
#include "kd_internal.h"

namespace kd {

constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;

// Router logits r[b][e] = W_r[e] . z[b] (fp32): one wave per (expert, row), grid (E, B).  Lane
// l adds float4 elements l, l + 64, ... of the row in order (kRouterVec of them in flight per
// pass), then the wave adds its lanes by a fixed butterfly: the order depends on d only.
constexpr int kRouterVec = 12;  // float4 per lane per pass: rows of up to 3072 in one pass
__global__ __launch_bounds__(64) void router_logits_kernel(const float* __restrict__ z, const float* __restrict__ Wr,
                                                           int d, int E, float* __restrict__ logits) {
  const int e = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const float4* w4 = reinterpret_cast<const float4*>(Wr + (size_t)e * d);
  const float4* z4 = reinterpret_cast<const float4*>(z + (size_t)b * d);
  const int d4 = d / 4;
  float acc = 0.0f;
  for (int base = 0; base < d4; base += 64 * kRouterVec) {
    float4 wv[kRouterVec], zv[kRouterVec];
#pragma unroll
    for (int i = 0; i < kRouterVec; ++i) {
      const int idx = base + lane + 64 * i;
      const bool ok = idx < d4;
      wv[i] = ok ? w4[idx] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      zv[i] = ok ? z4[idx] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int i = 0; i < kRouterVec; ++i) {
      acc = fmaf(wv[i].x, zv[i].x, acc);
      acc = fmaf(wv[i].y, zv[i].y, acc);
      acc = fmaf(wv[i].z, zv[i].z, acc);
      acc = fmaf(wv[i].w, zv[i].w, acc);
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) logits[(size_t)b * E + e] = acc;
}

// Top-K of every row and the expert buckets, in one workgroup of 16 waves.  Wave b takes row b:
// its lanes hold experts l + 64 i (NS slots), and each of K rounds takes the largest live logit
// (a float maximum, exact in any order: DPP within 16-lane rows, then the rows' maxima), then
// the lowest live expert id holding it (slot by slot, the first set bit of the first non-empty
// ballot), so ties go to the lower id.  Lane k keeps round k's logit and id; the softmax over
// the K selected logits adds their exponentials in rank order.  Then each wave lists, for its
// experts, the (row, rank) pairs routed there in ascending row order (ballots over the pairs).
template <int NS>
__global__ __launch_bounds__(1024) void route_bucket_kernel(const float* __restrict__ logits, int B, int E, int K,
                                                            int32_t* __restrict__ ids, float* __restrict__ p,
                                                            int32_t* __restrict__ count, int32_t* __restrict__ rows,
                                                            int32_t* __restrict__ pairs) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  __shared__ int32_t sids[KD_MAX_B * kMaxTopK];
  if (w < B) {
    float v[NS];
    bool live[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int e = lane + 64 * i;
      live[i] = e < E;
      v[i] = live[i] ? logits[(size_t)w * E + e] : 0.0f;
    }
    float myv = 0.0f;  // lane k < K: the logit and expert of rank k
    int mye = 0;
    for (int k = 0; k < K; ++k) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < NS; ++i) m = live[i] ? fmaxf(m, v[i]) : m;
      const float M = wave_max(m);
      int sel = -1;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const uint64_t bq = __ballot(live[i] && v[i] == M);
        if (sel < 0 && bq) sel = 64 * i + __builtin_ctzll(bq);
      }
      if (sel < 0) {  // no live logit equals the maximum (NaN logits only): the lowest live id
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const uint64_t bq = __ballot(live[i]);
          if (sel < 0 && bq) sel = 64 * i + __builtin_ctzll(bq);
        }
      }
      float vs = v[0];
#pragma unroll
      for (int i = 1; i < NS; ++i) vs = (sel >> 6) == i ? v[i] : vs;
      vs = lane_f(vs, sel & 63);
#pragma unroll
      for (int i = 0; i < NS; ++i) live[i] = live[i] && lane + 64 * i != sel;
      if (lane == k) {
        myv = vs;
        mye = sel;
      }
    }
    // p = softmax over the selected logits: exponentials per lane, their sum in rank order
    const float mx = lane_f(myv, 0);
    const float ex = lane < K ? expf(myv - mx) : 0.0f;
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) sum += lane_f(ex, k);
    if (lane < K) {
      ids[w * K + lane] = mye;
      p[w * K + lane] = ex / sum;
      sids[w * K + lane] = mye;
    }
  }
  __syncthreads();
  // one wave per expert: lane l looks at pairs l + 64 q (B K <= 256); a pair's place in its
  // expert's list is the number of matching pairs before it (ascending pair order)
  constexpr int kPairChunks = KD_MAX_B * kMaxTopK / 64;
  const int n = B * K, nq = (n + 63) / 64, nwv = blockDim.x >> 6;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int sj[kPairChunks], rj[kPairChunks];  // expert (-1 past the n pairs) and row of pair lane + 64 q
#pragma unroll
  for (int q = 0; q < kPairChunks; ++q) {
    sj[q] = q < nq && lane + 64 * q < n ? sids[lane + 64 * q] : -1;
    rj[q] = (lane + 64 * q) / K;
  }
  for (int e = w; e < E; e += nwv) {
    int c0 = 0;
#pragma unroll
    for (int q = 0; q < kPairChunks; ++q) {
      if (q >= nq) break;
      const int j = lane + 64 * q;
      const bool m = sj[q] == e;
      const uint64_t bq = __ballot(m);
      if (m) {
        const int c = c0 + __popcll(bq & below);
        rows[e * 16 + c] = rj[q];
        pairs[e * 16 + c] = j;
      }
      c0 += __popcll(bq);
    }
    if (lane == 0) count[e] = c0;
  }
}

void launch_router(const float* z, const float* Wr, int B, int d, int E, int K, int32_t* ids, float* p, float* logits,
                   int32_t* count, int32_t* rows, int32_t* pairs, hipStream_t st) {
  router_logits_kernel<<<dim3(E, B), 64, 0, st>>>(z, Wr, d, E, logits);
  switch (ceil_div(E, 64)) {
    case 1: route_bucket_kernel<1><<<1, 1024, 0, st>>>(logits, B, E, K, ids, p, count, rows, pairs); break;
    case 2: route_bucket_kernel<2><<<1, 1024, 0, st>>>(logits, B, E, K, ids, p, count, rows, pairs); break;
    case 3: route_bucket_kernel<3><<<1, 1024, 0, st>>>(logits, B, E, K, ids, p, count, rows, pairs); break;
    default: route_bucket_kernel<4><<<1, 1024, 0, st>>>(logits, B, E, K, ids, p, count, rows, pairs); break;
  }
}

int moe_max_experts() { return kMaxExperts; }
int moe_max_topk() { return kMaxTopK; }

}  // namespace kd

using namespace kd;

extern "C" kd_status kd_debug_moe_route(const float* z, const float* router, int32_t B, int32_t d, int32_t E,
                                        int32_t K, int32_t* ids, float* p, float* logits, int32_t* count,
                                        int32_t* rows, int32_t* pairs, void* stream) {
  const char* who = "kd_debug_moe_route";
  KD_REQUIRE(B >= 1 && B <= KD_MAX_B, KD_ERR_UNSUPPORTED, "%s: B=%d outside [1,16]", who, B);
  KD_REQUIRE(E >= 1 && E <= kMaxExperts && K >= 1 && K <= kMaxTopK && K <= E, KD_ERR_UNSUPPORTED,
             "%s: E=%d K=%d (E <= %d, K <= min(E, %d))", who, E, K, kMaxExperts, kMaxTopK);
  KD_REQUIRE(d > 0 && d % 4 == 0, KD_ERR_UNSUPPORTED, "%s: d=%d is not a positive multiple of 4", who, d);
  KD_REQUIRE(z && router && ids && p && logits && count && rows && pairs, KD_ERR_INVALID, "%s: null pointer", who);
  KD_REQUIRE(aligned16(z) && aligned16(router), KD_ERR_INVALID, "%s: z and router must be 16-byte aligned", who);
  launch_router(z, router, B, d, E, K, ids, p, logits, count, rows, pairs, as_stream(stream));
  return check_launch(who);
}
