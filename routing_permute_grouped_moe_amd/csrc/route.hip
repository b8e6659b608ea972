// Softmax top-k routing and its backward ([CANN-MoE] s2.1: Softmax -> Top-k
// -> mask, fused into one kernel).  One wavefront per token: each lane holds
// the logits of experts lane, lane+64, ...; the row max and the exp-sum are
// wave shuffle reductions, and the top k under the order (logit descending,
// expert index ascending) come from a radix select on ballots.
#include "validate.hpp"

#define ROUTE_WAVES 4           // tokens per workgroup
#define ROUTE_MAXV 16           // logits per lane: E <= 1024 (kernels are built for
                                // V = 1, 2, 4, 8, 16 logits per lane, the smallest
                                // with 64 V >= E is launched)

// Order-preserving key of a finite logit: larger logit <-> larger key; -0 is
// taken as +0 so that equal logits have equal keys (ties go by index).
__device__ __forceinline__ uint32_t route_key(float v) {
  uint32_t u = __float_as_uint(v);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k without cross-lane shuffles: the k-th largest key is found bit by bit
// from the top (a key bit is kept when at least k keys reach the prefix with
// it set; counts are wave ballots), the keys above it are chosen, and of the
// keys equal to it the ones with the lowest expert index fill the rest.  The
// slot of a chosen expert is the number of chosen experts ahead of it in the
// order (logit descending, index ascending) -- everything ahead of a chosen
// expert is chosen too.  Padding lanes (index >= E) hold key 0, below every
// finite logit's key, and k <= E.
template <int V>
__global__ __launch_bounds__(ROUTE_WAVES * MOE_WAVE) void route_fwd_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ idx,
    float* __restrict__ gate) {
  const int lane = threadIdx.x % MOE_WAVE;
  const int t = blockIdx.x * ROUTE_WAVES + threadIdx.x / MOE_WAVE;
  if (t >= T) return;
  const float* row = logits + (long long)t * E;
  float v[V];
  uint32_t key[V];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = lane + i * MOE_WAVE;
    v[i] = e < E ? row[e] : -INFINITY;
    key[i] = e < E ? route_key(v[i]) : 0u;
    m = fmaxf(m, v[i]);
  }
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = lane + i * MOE_WAVE;
    if (e < E) s += expf(v[i] - m);
  }
  s = wave_sum(s);
  const float inv = 1.0f / s;
  // the k-th largest key
  uint32_t K = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = K | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) cnt += __popcll(__ballot(key[i] >= c));
    if (cnt >= k) K = c;
  }
  // chosen: keys above K, then ties at K by ascending index (i, then lane)
  int need = k;
#pragma unroll
  for (int i = 0; i < V; ++i) need -= __popcll(__ballot(key[i] > K));
  const unsigned long long below = (1ull << lane) - 1ull;
  bool sel[V];
  unsigned long long bsel[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const unsigned long long tie = __ballot(key[i] == K);
    sel[i] = key[i] > K || (key[i] == K && __popcll(tie & below) < need);
    const int nt = __popcll(tie);
    need -= need < nt ? need : nt;
    bsel[i] = __ballot(sel[i]);
  }
  // slots: chosen experts ahead of each chosen one
  int slot[V];
#pragma unroll
  for (int i = 0; i < V; ++i) slot[i] = 0;
#pragma unroll
  for (int i2 = 0; i2 < V; ++i2) {
    unsigned long long bm = bsel[i2];
    while (bm) {
      const int l2 = __builtin_ctzll(bm);
      bm &= bm - 1;
      const uint32_t k2 = (uint32_t)__builtin_amdgcn_readlane((int)key[i2], l2);
      const int e2 = l2 + i2 * MOE_WAVE;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int e = lane + i * MOE_WAVE;
        slot[i] += (k2 > key[i]) || (k2 == key[i] && e2 < e);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < V; ++i)
    if (sel[i]) {
      const int e = lane + i * MOE_WAVE;
      idx[(long long)t * k + slot[i]] = e;
      gate[(long long)t * k + slot[i]] = expf(v[i] - m) * inv;
    }
}

template <int V>
__global__ __launch_bounds__(ROUTE_WAVES * MOE_WAVE) void route_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ dgate, int T, int E, int k, float* __restrict__ dlogits) {
  __shared__ float dp_s[ROUTE_WAVES][MOE_MAX_E];
  const int lane = threadIdx.x % MOE_WAVE;
  const int w = threadIdx.x / MOE_WAVE;
  const int t = blockIdx.x * ROUTE_WAVES + w;
  if (t >= T) return;  // whole wave leaves together; no block barrier below
  const float* row = logits + (long long)t * E;
  float* dp = dp_s[w];
  for (int e = lane; e < E; e += MOE_WAVE) dp[e] = 0.f;
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  // chosen experts of a token are distinct, so these writes never collide
  for (int j = lane; j < k; j += MOE_WAVE) {
    int e = idx[(long long)t * k + j];
    if (e >= 0 && e < E) dp[e] = dgate[(long long)t * k + j];
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  float v[V];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    int e = lane + i * MOE_WAVE;
    v[i] = e < E ? row[e] : -INFINITY;
    m = fmaxf(m, v[i]);
  }
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    int e = lane + i * MOE_WAVE;
    v[i] = e < E ? expf(v[i] - m) : 0.f;
    s += v[i];
  }
  s = wave_sum(s);
  const float inv = 1.0f / s;
  float acc = 0.f;  // sum_e p_e dp_e
#pragma unroll
  for (int i = 0; i < V; ++i) {
    int e = lane + i * MOE_WAVE;
    if (e < E) acc += v[i] * inv * dp[e];
  }
  acc = wave_sum(acc);
#pragma unroll
  for (int i = 0; i < V; ++i) {
    int e = lane + i * MOE_WAVE;
    if (e < E) dlogits[(long long)t * E + e] = v[i] * inv * (dp[e] - acc);
  }
}

// logits per lane of the kernel launched for E experts
static int route_width(int E) {
  int v = 1;
  while (v * MOE_WAVE < E && v < ROUTE_MAXV) v *= 2;
  return v;
}

template <int V>
static void launch_fwd(dim3 grid, hipStream_t s, const float* logits, int T, int E, int k,
                       int32_t* idx, float* gate) {
  hipLaunchKernelGGL(route_fwd_kernel<V>, grid, dim3(ROUTE_WAVES * MOE_WAVE), 0, s, logits, T, E,
                     k, idx, gate);
}
template <int V>
static void launch_bwd(dim3 grid, hipStream_t s, const float* logits, const int32_t* idx,
                       const float* dgate, int T, int E, int k, float* dlogits) {
  hipLaunchKernelGGL(route_bwd_kernel<V>, grid, dim3(ROUTE_WAVES * MOE_WAVE), 0, s, logits, idx,
                     dgate, T, E, k, dlogits);
}

extern "C" int moe_route(const float* logits, int T, int E, int k, int32_t* idx, float* gate,
                         moe_stream_t stream) {
  const char* fn = "moe_route";
  MOE_TRY(moe_need_nonneg(T, fn, "T"));
  MOE_TRY(moe_need_ek(E, k, fn));
  if (T == 0) return MOE_OK;
  MOE_TRY(moe_need_ptr(logits, fn, "logits", 4));
  MOE_TRY(moe_need_ptr(idx, fn, "idx", 4));
  MOE_TRY(moe_need_ptr(gate, fn, "gate", 4));
  MOE_TRY(moe_need_elems(T, E, 4, fn, "logits"));
  dim3 grid((T + ROUTE_WAVES - 1) / ROUTE_WAVES);
  hipStream_t s = (hipStream_t)stream;
  switch (route_width(E)) {
    case 1: launch_fwd<1>(grid, s, logits, T, E, k, idx, gate); break;
    case 2: launch_fwd<2>(grid, s, logits, T, E, k, idx, gate); break;
    case 4: launch_fwd<4>(grid, s, logits, T, E, k, idx, gate); break;
    case 8: launch_fwd<8>(grid, s, logits, T, E, k, idx, gate); break;
    default: launch_fwd<16>(grid, s, logits, T, E, k, idx, gate); break;
  }
  return moe_check_launch(fn);
}

extern "C" int moe_route_bwd(const float* logits, const int32_t* idx, const float* dgate, int T,
                             int E, int k, float* dlogits, moe_stream_t stream) {
  const char* fn = "moe_route_bwd";
  MOE_TRY(moe_need_nonneg(T, fn, "T"));
  MOE_TRY(moe_need_ek(E, k, fn));
  if (T == 0) return MOE_OK;
  MOE_TRY(moe_need_ptr(logits, fn, "logits", 4));
  MOE_TRY(moe_need_ptr(idx, fn, "idx", 4));
  MOE_TRY(moe_need_ptr(dgate, fn, "dgate", 4));
  MOE_TRY(moe_need_ptr(dlogits, fn, "dlogits", 4));
  MOE_TRY(moe_need_elems(T, E, 4, fn, "logits"));
  dim3 grid((T + ROUTE_WAVES - 1) / ROUTE_WAVES);
  hipStream_t s = (hipStream_t)stream;
  switch (route_width(E)) {
    case 1: launch_bwd<1>(grid, s, logits, idx, dgate, T, E, k, dlogits); break;
    case 2: launch_bwd<2>(grid, s, logits, idx, dgate, T, E, k, dlogits); break;
    case 4: launch_bwd<4>(grid, s, logits, idx, dgate, T, E, k, dlogits); break;
    case 8: launch_bwd<8>(grid, s, logits, idx, dgate, T, E, k, dlogits); break;
    default: launch_bwd<16>(grid, s, logits, idx, dgate, T, E, k, dlogits); break;
  }
  return moe_check_launch(fn);
}
