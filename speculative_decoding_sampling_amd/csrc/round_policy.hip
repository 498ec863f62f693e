// Round statistics and the adaptive draft length, kept on the device so that
// a decode loop needs no host round trip between rounds.
//
// tbxsx.cn "推测解码采样验证优化策略 —— 深度调研报告", section "4. 实现逻辑":
// after each round an acceptance-rate monitor with a window of rounds takes
// the round's accepted and drafted counts, and the draft length K moves up by
// one (at most the maximum draft length) when the rate is above 0.85 and down
// by one (at least 1) when it is below 0.60.  nickwang.xyz
// "推测解码：草稿、验证与实际加速", section "好草稿也要算得便宜": E[N] tokens per
// round from the acceptance rates, and the tokens a round really commits.
//
// Every request of a batch is its own sequence with its own window.  The
// monitor state is plain integers, so the rule is decided exactly: the rate
// a/d is compared with 17/20 and 3/5 by cross-multiplication.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kPolicyThreads = 256;
constexpr int kStatsThreads = 1024;
constexpr int kNumTotals = 8;

// Accepted drafts of request b's round, or -1 for a failed round.  The
// first n - 1 emitted tokens are accepted drafts; the last one is too only
// when the round stopped on an accepted EOS, i.e. it sits at a drafted
// position and equals the draft there.  A correction cannot equal the
// rejected draft: the residual max(p - q, 0) is zero at a token whose ratio
// p/q was below one.
__device__ __forceinline__ int accepted_drafts(const int32_t* __restrict__ draft_tokens,
                                               const int32_t* __restrict__ out_tokens, int b,
                                               int K, int nb, int n) {
  if (nb < 0 || nb > K || n < 1 || n > nb + 1) return -1;
  const int last = n - 1;
  if (last < nb && out_tokens[(size_t)b * (K + 1) + last] == draft_tokens[(size_t)b * K + last])
    return n;
  return n - 1;
}

// Totals: requests, errors, drafted, accepted, emitted, eos_stops,
// full_accepts, rejections.  With totals the grid is one workgroup.
__global__ __launch_bounds__(kStatsThreads) void round_stats_kernel(
    const int32_t* __restrict__ draft_tokens, const int32_t* __restrict__ draft_len,
    const int32_t* __restrict__ out_tokens, const int32_t* __restrict__ n_emitted,
    const float* __restrict__ beta, int B, int K, int32_t* __restrict__ accepted,
    float* __restrict__ expected, long long* __restrict__ totals) {
  long long t[kNumTotals] = {};
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < B; b += gridDim.x * blockDim.x) {
    const int nb = draft_len[b], n = n_emitted[b];
    const int a = accepted_drafts(draft_tokens, out_tokens, b, K, nb, n);
    if (accepted) accepted[b] = a;
    if (a < 0) {
      t[1] += 1;
    } else {
      t[0] += 1;
      t[2] += nb;
      t[3] += a;
      t[4] += n;
      t[a == n ? 5 : a == nb ? 6 : 7] += 1;
    }
    if (expected) {
      // 1 + beta_0 + beta_0 beta_1 + ...: independent positions, each with
      // its own rate.  Rounded products and sums, no fused steps, in order.
      double total = -1.0;
      if (nb >= 0 && nb <= K) {
        double run = 1.0;
        total = 1.0;
        for (int k = 0; k < nb; ++k) {
          const float r = beta[(size_t)b * K + k];
          if (!(r >= 0.f)) { total = -1.0; break; }
          run = __dmul_rn(run, (double)r);
          total = __dadd_rn(total, run);
        }
      }
      expected[b] = (float)total;
    }
  }
  if (!totals) return;
  __shared__ long long red[kStatsThreads / 64][kNumTotals];
  const int lane = threadIdx.x % 64, wid = threadIdx.x / 64;
#pragma unroll
  for (int i = 0; i < kNumTotals; ++i) {
    long long v = t[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) red[wid][i] = v;
  }
  __syncthreads();
  if (threadIdx.x < kNumTotals) {
    long long s = 0;
    for (int w = 0; w < (int)(blockDim.x / 64); ++w) s += red[w][threadIdx.x];
    totals[threadIdx.x] = s;
  }
}

// Monitor state of one request, int32: head, filled, window sums of accepted
// drafts and of drafted positions, then the ring of the last `window` rounds,
// each packed as accepted | drafted << 16.
__host__ __device__ constexpr size_t monitor_stride(int window) {
  return ((size_t)4 + (size_t)window + 3) / 4 * 4;
}

__global__ __launch_bounds__(kPolicyThreads) void monitor_reset_kernel(int4* __restrict__ state,
                                                                      size_t n4) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x)
    state[i] = make_int4(0, 0, 0, 0);
}

__global__ __launch_bounds__(kPolicyThreads) void monitor_update_kernel(
    const int32_t* __restrict__ draft_tokens, const int32_t* draft_len,
    const int32_t* __restrict__ out_tokens, const int32_t* __restrict__ n_emitted, int B, int K,
    int max_k, int window, int32_t* __restrict__ state, int32_t* next_draft_len,
    double* __restrict__ rate) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int32_t* st = state + (size_t)b * monitor_stride(window);
  int4 h = *reinterpret_cast<const int4*>(st);        // head, filled, sum_acc, sum_drafted
  // A header no reset wrote (or one for another window) would index outside
  // the ring: such a window starts again empty.
  if (h.x < 0 || h.x >= window || h.y < 0 || h.y > window || h.z < 0 || h.w < 0 || h.z > h.w)
    h = make_int4(0, 0, 0, 0);
  const int nb = draft_len[b];
  const int a = accepted_drafts(draft_tokens, out_tokens, b, K, nb, n_emitted[b]);
  if (a >= 0) {                                       // a failed round adds nothing
    int32_t* ring = st + 4;
    if (h.y == window) {
      const int old = ring[h.x];
      h.z -= old & 0xffff;
      h.w -= old >> 16;
    } else {
      h.y += 1;
    }
    ring[h.x] = a | (nb << 16);
    h.x = h.x + 1 == window ? 0 : h.x + 1;
    h.z += a;
    h.w += nb;
    *reinterpret_cast<int4*>(st) = h;
  }
  int k = nb;
  if (h.w > 0) {
    const long long acc = h.z, drafted = h.w;
    if (20 * acc > 17 * drafted) k = k + 1;            // rate > 17/20
    else if (5 * acc < 3 * drafted) k = k - 1;         // rate < 3/5
  }
  k = k < 1 ? 1 : (k > max_k ? max_k : k);
  if (rate) rate[b] = h.w > 0 ? (double)h.z / (double)h.w : -1.0;
  next_draft_len[b] = k;                              // may alias draft_len: read above
}

hipError_t launch_round_stats(const int32_t* draft_tokens, const int32_t* draft_len,
                              const int32_t* out_tokens, const int32_t* n_emitted,
                              const float* beta, int B, int K, int32_t* accepted, float* expected,
                              long long* totals, hipStream_t stream) {
  const int blocks = totals ? 1 : (B + kStatsThreads - 1) / kStatsThreads;
  round_stats_kernel<<<dim3(blocks), dim3(kStatsThreads), 0, stream>>>(
      draft_tokens, draft_len, out_tokens, n_emitted, beta, B, K, accepted, expected, totals);
  return hipGetLastError();
}

size_t monitor_state_bytes(int B, int window) {
  return (size_t)B * monitor_stride(window) * sizeof(int32_t);
}

hipError_t launch_monitor_reset(void* state, int B, int window, hipStream_t stream) {
  const size_t n4 = (size_t)B * monitor_stride(window) / 4;
  size_t blocks = (n4 + kPolicyThreads - 1) / kPolicyThreads;
  if (blocks > 4096) blocks = 4096;
  monitor_reset_kernel<<<dim3((unsigned)blocks), dim3(kPolicyThreads), 0, stream>>>(
      static_cast<int4*>(state), n4);
  return hipGetLastError();
}

hipError_t launch_monitor_update(const int32_t* draft_tokens, const int32_t* draft_len,
                                 const int32_t* out_tokens, const int32_t* n_emitted, int B,
                                 int K, int max_k, int window, void* state,
                                 int32_t* next_draft_len, double* rate, hipStream_t stream) {
  monitor_update_kernel<<<dim3((B + kPolicyThreads - 1) / kPolicyThreads), dim3(kPolicyThreads),
                          0, stream>>>(draft_tokens, draft_len, out_tokens, n_emitted, B, K,
                                       max_k, window, static_cast<int32_t*>(state),
                                       next_draft_len, rate);
  return hipGetLastError();
}

}  // namespace specv
