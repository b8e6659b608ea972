// Router projection in fp32 ([CANN-MoE] s4.2 keeps the router in FP32) and
// its backward.  The three products are small next to the expert GEMMs
// (N = E or K = E), so they use one strided fp32 tile kernel:
//   C[m,n] = sum_k A(m,k) B(k,n) (+ bias[n])
// A(m,k) = A[m*a_sm + k*a_sk] (storage type TA, widened to fp32),
// B(k,n) = B[k*b_sk + n*b_sn] (fp32).  64x64 tile per 256-thread block,
// 4x4 outputs per thread, K staged through LDS 16 at a time.
#include "validate.hpp"

#define RT_BM 64
#define RT_BN 64
#define RT_BK 16

template <typename TA> __device__ __forceinline__ float ld_as_f32(const TA* p, long long i);
template <> __device__ __forceinline__ float ld_as_f32<float>(const float* p, long long i) {
  return p[i];
}
template <> __device__ __forceinline__ float ld_as_f32<bf16_t>(const bf16_t* p, long long i) {
  return bf16_to_f32(p[i]);
}
template <typename TC> __device__ __forceinline__ void st_from_f32(TC* p, long long i, float v);
template <> __device__ __forceinline__ void st_from_f32<float>(float* p, long long i, float v) {
  p[i] = v;
}
template <> __device__ __forceinline__ void st_from_f32<bf16_t>(bf16_t* p, long long i, float v) {
  p[i] = (bf16_t)f32_to_bf16(v);
}

template <typename TA, typename TC>
__global__ __launch_bounds__(256) void router_gemm_kernel(
    const TA* __restrict__ A, long long a_sm, long long a_sk, const float* __restrict__ B,
    long long b_sk, long long b_sn, const float* __restrict__ bias, int M, int N, int K,
    TC* __restrict__ C, long long c_sm) {
  __shared__ float As[RT_BK][RT_BM + 4];
  __shared__ float Bs[RT_BK][RT_BN + 4];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * RT_BM, n0 = blockIdx.x * RT_BN;
  const int tm = (tid / 16) * 4, tn = (tid % 16) * 4;
  // Each K step of 16 is summed on its own, then added to the running sum with
  // Kahan compensation, so the rounding error does not grow with K (K is up
  // to H = 7680 for the logits and T for dWg); it keeps near-equal logits in
  // the right order.
  float acc[4][4] = {}, comp[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += RT_BK) {
    // 64x16 A values and 16x64 B values, 4 each per thread
    for (int i = tid; i < RT_BM * RT_BK; i += 256) {
      int mm, kk;
      if (a_sk == 1) { mm = i / RT_BK; kk = i % RT_BK; } else { kk = i / RT_BM; mm = i % RT_BM; }
      int m = m0 + mm, kq = k0 + kk;
      As[kk][mm] = (m < M && kq < K) ? ld_as_f32<TA>(A, m * a_sm + kq * a_sk) : 0.f;
    }
    for (int i = tid; i < RT_BN * RT_BK; i += 256) {
      int nn, kk;
      if (b_sn == 1) { kk = i / RT_BN; nn = i % RT_BN; } else { nn = i / RT_BK; kk = i % RT_BK; }
      int n = n0 + nn, kq = k0 + kk;
      Bs[kk][nn] = (n < N && kq < K) ? B[kq * b_sk + n * b_sn] : 0.f;
    }
    __syncthreads();
    float part[4][4] = {};
#pragma unroll
    for (int kk = 0; kk < RT_BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][tm + i]; b[i] = Bs[kk][tn + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) part[i][j] = fmaf(a[i], b[j], part[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float y = part[i][j] - comp[i][j];
        const float t = acc[i][j] + y;
        comp[i][j] = (t - acc[i][j]) - y;
        acc[i][j] = t;
      }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = m0 + tm + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int n = n0 + tn + j;
      if (n >= N) continue;
      float v = acc[i][j] + (bias ? bias[n] : 0.f);
      st_from_f32<TC>(C, m * c_sm + n, v);
    }
  }
}

// dbias[e] = sum_t dl[t,e]; 64 columns x 16 row slices per block, fixed order.
__global__ __launch_bounds__(1024) void colsum_kernel(const float* __restrict__ dl, int T, int E,
                                                      float* __restrict__ out) {
  __shared__ float part[16][MOE_WAVE];
  const int lane = threadIdx.x % MOE_WAVE, s = threadIdx.x / MOE_WAVE;
  const int e = blockIdx.x * MOE_WAVE + lane;
  const int per = (T + 15) / 16;
  float sum = 0.f;
  if (e < E)
    for (int t = s * per; t < min(T, (s + 1) * per); ++t) sum += dl[(long long)t * E + e];
  part[s][lane] = sum;
  __syncthreads();
  if (s == 0 && e < E) {
    float tot = 0.f;
    for (int i = 0; i < 16; ++i) tot += part[i][lane];
    out[e] = tot;
  }
}

template <typename TA, typename TC>
static void launch_router_gemm(hipStream_t s, const TA* A, long long a_sm, long long a_sk,
                               const float* B, long long b_sk, long long b_sn, const float* bias,
                               int M, int N, int K, TC* C, long long c_sm) {
  dim3 grid((N + RT_BN - 1) / RT_BN, (M + RT_BM - 1) / RT_BM);
  hipLaunchKernelGGL((router_gemm_kernel<TA, TC>), grid, dim3(256), 0, s, A, a_sm, a_sk, B, b_sk,
                     b_sn, bias, M, N, K, C, c_sm);
}

static int router_checks(const char* fn, int dt, int T, int H, int E) {
  MOE_TRY(moe_need_dt(dt, fn));
  MOE_TRY(moe_need_nonneg(T, fn, "T"));
  MOE_TRY(moe_need_mult64(H, fn, "H"));
  MOE_TRY(moe_need_ek(E, 1, fn));
  MOE_TRY(moe_need_elems(T, H, moe_dt_bytes(dt), fn, "x"));
  MOE_TRY(moe_need_elems(T, E, 4, fn, "logits"));
  return MOE_OK;
}

extern "C" int moe_router_logits(const void* x, int dt, const float* wg, const float* bias, int T,
                                 int H, int E, float* logits, moe_stream_t stream) {
  const char* fn = "moe_router_logits";
  MOE_TRY(router_checks(fn, dt, T, H, E));
  if (T == 0) return MOE_OK;
  MOE_TRY(moe_need_ptr(x, fn, "x"));
  MOE_TRY(moe_need_ptr(wg, fn, "wg", 4));
  MOE_TRY(moe_opt_ptr(bias, fn, "bias", 4));
  MOE_TRY(moe_need_ptr(logits, fn, "logits", 4));
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOE_BF16)
    launch_router_gemm<bf16_t, float>(s, (const bf16_t*)x, H, 1, wg, E, 1, bias, T, E, H, logits, E);
  else
    launch_router_gemm<float, float>(s, (const float*)x, H, 1, wg, E, 1, bias, T, E, H, logits, E);
  return moe_check_launch(fn);
}

extern "C" int moe_router_logits_bwd(const float* dlogits, const void* x, int dt, const float* wg,
                                     int T, int H, int E, void* dx, float* dwg, float* dbias,
                                     moe_stream_t stream) {
  const char* fn = "moe_router_logits_bwd";
  MOE_TRY(router_checks(fn, dt, T, H, E));
  MOE_TRY(moe_need_ptr(dwg, fn, "dwg", 4));
  MOE_TRY(moe_opt_ptr(dbias, fn, "dbias", 4));
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {
    // no tokens: the weight gradients are zero
    hipLaunchKernelGGL((router_gemm_kernel<float, float>), dim3((E + RT_BN - 1) / RT_BN, (H + RT_BM - 1) / RT_BM),
                       dim3(256), 0, s, (const float*)nullptr, 0LL, 0LL, (const float*)nullptr, 0LL,
                       0LL, (const float*)nullptr, H, E, 0, dwg, (long long)E);
    if (dbias)
      hipLaunchKernelGGL(colsum_kernel, dim3((E + MOE_WAVE - 1) / MOE_WAVE), dim3(1024), 0, s,
                         (const float*)nullptr, 0, E, dbias);
    return moe_check_launch(fn);
  }
  MOE_TRY(moe_need_ptr(dlogits, fn, "dlogits", 4));
  MOE_TRY(moe_need_ptr(x, fn, "x"));
  MOE_TRY(moe_need_ptr(wg, fn, "wg", 4));
  MOE_TRY(moe_need_ptr(dx, fn, "dx"));
  // dx[T,H] = dlogits[T,E] . Wg^T : B(k=e, n=h) = Wg[h*E + e]
  if (dt == MOE_BF16)
    launch_router_gemm<float, bf16_t>(s, dlogits, E, 1, wg, 1, E, nullptr, T, H, E, (bf16_t*)dx, H);
  else
    launch_router_gemm<float, float>(s, dlogits, E, 1, wg, 1, E, nullptr, T, H, E, (float*)dx, H);
  MOE_TRY(moe_check_launch(fn));
  // dWg[H,E] = x^T . dlogits : A(m=h, k=t) = x[t*H + h]
  if (dt == MOE_BF16)
    launch_router_gemm<bf16_t, float>(s, (const bf16_t*)x, 1, H, dlogits, E, 1, nullptr, H, E, T,
                                      dwg, E);
  else
    launch_router_gemm<float, float>(s, (const float*)x, 1, H, dlogits, E, 1, nullptr, H, E, T, dwg,
                                     E);
  MOE_TRY(moe_check_launch(fn));
  if (dbias) {
    hipLaunchKernelGGL(colsum_kernel, dim3((E + MOE_WAVE - 1) / MOE_WAVE), dim3(1024), 0, s,
                       dlogits, T, E, dbias);
    MOE_TRY(moe_check_launch(fn));
  }
  return MOE_OK;
}
