// Softmax top-k routing and its backward ([CANN-MoE] s2.1: Softmax -> Top-k
// -> mask, fused into one kernel).  One wavefront per token: each lane holds
// the logits of experts lane, lane+64, ...; the row max and the exp-sum are
// wave shuffle reductions, and each of the k selections is a wave arg-max
// under the order (logit descending, expert index ascending).
#include "validate.hpp"

#define ROUTE_WAVES 4           // tokens per workgroup
#define ROUTE_MAXV 16           // logits per lane: E <= 1024 (kernels are built for
                                // V = 1, 2, 4, 8, 16 logits per lane, the smallest
                                // with 64 V >= E is launched)

__device__ __forceinline__ bool route_better(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
}

template <int V>
__global__ __launch_bounds__(ROUTE_WAVES * MOE_WAVE) void route_fwd_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ idx,
    float* __restrict__ gate) {
  const int lane = threadIdx.x % MOE_WAVE;
  const int t = blockIdx.x * ROUTE_WAVES + threadIdx.x / MOE_WAVE;
  if (t >= T) return;
  const float* row = logits + (long long)t * E;
  float v[V];
  bool taken[V];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    int e = lane + i * MOE_WAVE;
    v[i] = e < E ? row[e] : -INFINITY;
    taken[i] = e >= E;
    m = fmaxf(m, v[i]);
  }
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    int e = lane + i * MOE_WAVE;
    if (e < E) s += expf(v[i] - m);
  }
  s = wave_sum(s);
  const float inv = 1.0f / s;
  for (int j = 0; j < k; ++j) {
    // best candidate of this lane
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      int e = lane + i * MOE_WAVE;
      if (!taken[i] && route_better(v[i], e, bv, be)) { bv = v[i]; be = e; }
    }
    // wave arg-max
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float ov = __shfl_xor(bv, o, MOE_WAVE);
      int oe = __shfl_xor(be, o, MOE_WAVE);
      if (route_better(ov, oe, bv, be)) { bv = ov; be = oe; }
    }
    // be is now the same in every lane; the owner marks it taken
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (lane + i * MOE_WAVE == be) taken[i] = true;
    if (lane == 0) {
      idx[(long long)t * k + j] = be;
      gate[(long long)t * k + j] = expf(bv - m) * inv;
    }
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
