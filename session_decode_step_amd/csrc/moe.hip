// Mixture-of-experts FFN for a batch of rows with experts merged across rows.
//
// What is computed (hf2q ADR-040 §0.7 F4: per-token top-k routing, rows grouped by expert so
// each active expert's weights are read once and applied to every row routed to it, then a
// per-row weighted sum; Strata pull request #1524 "What changes": merged expert execution
// and a shared expert): r = W_r z (fp32 router), the top-k experts by descending logit
// (ties to the lower id), p = softmax over the k selected logits, moe_b = sum_k p_k
// Expert_{e_k}(z_b) in rank order, plus the shared expert's output.
//
// How: routing and grouping run on the device (no host round trip).  The bucketing kernel
// lists, for each expert, the (row, rank) pairs routed to it in ascending row order; the
// grouped mmvq reads each active expert's tiles once (empty experts exit before reading)
// and treats its rows as the MFMA's activation rows, whose results never depend on which
// other rows share the expert; the combine adds the k expert outputs of a row in rank
// order.  So a row's result is the same at any B.
#include "kd_internal.h"

namespace kd {

constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;

// grid B; 256 threads.  z fp32 [B][d]; Wr fp32 [E][d].
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ z, const float* __restrict__ Wr,
                                                          int d, int E, int K, int32_t* __restrict__ ids,
                                                          float* __restrict__ p, float* __restrict__ logits) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  __shared__ float r[kMaxExperts];
  const float* zr = z + (size_t)b * d;
  for (int e = w; e < E; e += 4) {
    const float* wr = Wr + (size_t)e * d;
    float acc = 0.0f;
    for (int i = lane; i < d; i += 64) acc = fmaf(wr[i], zr[i], acc);
    acc = wave_sum(acc);
    if (lane == 0) r[e] = acc;
  }
  __syncthreads();
  if (logits)
    for (int e = tid; e < E; e += 256) logits[(size_t)b * E + e] = r[e];
  if (tid == 0) {
    bool taken[kMaxExperts];
    for (int e = 0; e < E; ++e) taken[e] = false;
    int sel[kMaxTopK];
    float val[kMaxTopK];
    for (int k = 0; k < K; ++k) {
      int best = -1;
      float bv = -INFINITY;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || r[e] > bv)) {  // strict: ties keep the lower id
          best = e;
          bv = r[e];
        }
      taken[best] = true;
      sel[k] = best;
      val[k] = bv;
    }
    const float mx = val[0];
    float ex[kMaxTopK];
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) {
      ex[k] = expf(val[k] - mx);
      sum += ex[k];
    }
    for (int k = 0; k < K; ++k) {
      ids[b * K + k] = sel[k];
      p[b * K + k] = ex[k] / sum;
    }
  }
}

// 1 workgroup, one thread per expert: rows routed to expert e, ascending row order.
__global__ void moe_bucket_kernel(const int32_t* __restrict__ ids, int B, int K, int E, int32_t* __restrict__ count,
                                  int32_t* __restrict__ rows, int32_t* __restrict__ pairs) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
    for (int b = 0; b < B; ++b)
      for (int k = 0; k < K; ++k)
        if (ids[b * K + k] == e) {
          rows[e * 16 + c] = b;
          pairs[e * 16 + c] = b * K + k;
          ++c;
        }
    count[e] = c;
  }
}

// f[b][i] = sum_k p[b][k] y[b*K + k][i] (rank order) + sh[b][i].
__global__ void moe_combine_kernel(const float* __restrict__ y, const float* __restrict__ p, const float* __restrict__ sh,
                                   int B, int K, int d, float* __restrict__ f) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * d) return;
  const int b = idx / d, i = idx % d;
  float acc = 0.0f;
  for (int k = 0; k < K; ++k) acc = fmaf(p[b * K + k], y[(size_t)(b * K + k) * d + i], acc);
  f[idx] = acc + sh[idx];
}

void launch_router(const float* z, const float* Wr, int B, int d, int E, int K, int32_t* ids, float* p, float* logits,
                   hipStream_t st) {
  router_topk_kernel<<<B, 256, 0, st>>>(z, Wr, d, E, K, ids, p, logits);
}

void launch_bucket(const int32_t* ids, int B, int K, int E, int32_t* count, int32_t* rows, int32_t* pairs,
                   hipStream_t st) {
  moe_bucket_kernel<<<1, 256, 0, st>>>(ids, B, K, E, count, rows, pairs);
}

void launch_moe_combine(const float* y, const float* p, const float* sh, int B, int K, int d, float* f, hipStream_t st) {
  moe_combine_kernel<<<ceil_div(B * d, 256), 256, 0, st>>>(y, p, sh, B, K, d, f);
}

int moe_max_experts() { return kMaxExperts; }
int moe_max_topk() { return kMaxTopK; }

}  // namespace kd
