// Router projection in fp32 ([CANN-MoE] s4.2 keeps the router in FP32) and
// its backward.
//
// bf16 tokens (H a multiple of 256, T a multiple of 256, E a multiple of 64)
// take the MFMA path: the fp32 operand (Wg, or dlogits for dWg) is split into
// three bf16 parts hi + mid + lo that carry all of its 24 mantissa bits; a
// product of a bf16 token value with each part is exact in fp32, the grouped
// GEMM kernel sums them over S = 8 K slices with fp32 accumulation, and the
// slices are added in fp64.  The input gradient dx only needs bf16 accuracy
// (it is stored in bf16) and uses the hi parts alone.
//
// Other shapes use one strided fp32 tile kernel:
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

// ---------------------------------------------------------------- MFMA path helpers

#define RT_SPLIT 8   // K slices of the router products

static bool mfma_path(int dt, int T, int H, int E) {
  // each K slice a whole number of the grouped GEMM's 32-deep bf16 K steps
  return dt == MOE_BF16 && H % (RT_SPLIT * 32) == 0 && T % (RT_SPLIT * 32) == 0 && E % 64 == 0;
}

// three bf16 parts of an fp32 value: hi = bf16(v), mid = bf16(v - hi),
// lo = bf16(v - hi - mid) (each difference is exact in fp32)
__device__ __forceinline__ void split3(float v, uint32_t& h, uint32_t& m, uint32_t& l) {
  h = f32_to_bf16(v);
  const float r1 = v - bf16_to_f32(h);
  m = f32_to_bf16(r1);
  l = f32_to_bf16(r1 - bf16_to_f32(m));
}

// The K rows of slice s are taken 32 at a time (one K step of the GEMM):
// the hi, mid and lo parts of a 32-row chunk follow each other, so the GEMM
// reads each 32-deep step of its token operand once and multiplies it by the
// three parts in consecutive K steps (krep = 3) while the step is in cache.
#define RT_CHUNK 32

// Wg [H,E] -> wg3s [S][H/S/32][3][32][E] and wgb [H,E] = hi part.
__global__ __launch_bounds__(256) void split_wg_kernel(const float* __restrict__ wg, int H, int E,
                                                       bf16_t* __restrict__ wg3s,
                                                       bf16_t* __restrict__ wgb) {
  const long long n = (long long)H * E;
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const int h = (int)(i / E), e = (int)(i % E);
    uint32_t p0, p1, p2;
    split3(wg[i], p0, p1, p2);
    const long long base = ((long long)(h - h % RT_CHUNK) * 3 + h % RT_CHUNK) * E + e;
    wg3s[base] = (bf16_t)p0;
    wg3s[base + RT_CHUNK * E] = (bf16_t)p1;
    wg3s[base + 2 * RT_CHUNK * E] = (bf16_t)p2;
    if (wgb) wgb[i] = (bf16_t)p0;
  }
}

// dl [T,E] -> dl3s [S][T/S/32][3][32][E] and dlb [T,E] = hi part.
__global__ __launch_bounds__(256) void split_dl_kernel(const float* __restrict__ dl, int T, int E,
                                                       bf16_t* __restrict__ dl3s,
                                                       bf16_t* __restrict__ dlb) {
  const long long n = (long long)T * E;
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const int t = (int)(i / E), e = (int)(i % E);
    uint32_t p0, p1, p2;
    split3(dl[i], p0, p1, p2);
    const long long base = ((long long)(t - t % RT_CHUNK) * 3 + t % RT_CHUNK) * E + e;
    dl3s[base] = (bf16_t)p0;
    dl3s[base + RT_CHUNK * E] = (bf16_t)p1;
    dl3s[base + 2 * RT_CHUNK * E] = (bf16_t)p2;
    dlb[i] = (bf16_t)p0;
  }
}

// out[i] = (bias[i % E]) + sum_s part[s][i], summed in fp64 in slice order.
__global__ __launch_bounds__(256) void reduce_slices_kernel(const float* __restrict__ part,
                                                            long long n, int E,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ out) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    double acc = bias ? (double)bias[i % E] : 0.0;
#pragma unroll
    for (int s = 0; s < RT_SPLIT; ++s) acc += (double)part[s * n + i];
    out[i] = (float)acc;
  }
}

// dbias: per-chunk column sums (COLSUM_ROWS tokens per chunk), then a fixed-order sum.
#define COLSUM_ROWS 64   // rows of one column partial sum
__global__ __launch_bounds__(256) void colsum_part_kernel(const float* __restrict__ dl, int T,
                                                          int E, float* __restrict__ part) {
  const int e = blockIdx.y * 256 + threadIdx.x;
  const int c = blockIdx.x;
  if (e >= E) return;
  const int t0 = c * COLSUM_ROWS;
  // all rows requested together, then added in row order
  float v[COLSUM_ROWS];
#pragma unroll
  for (int i = 0; i < COLSUM_ROWS; ++i) v[i] = t0 + i < T ? dl[(long long)(t0 + i) * E + e] : 0.f;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < COLSUM_ROWS; ++i) s += v[i];
  part[(long long)c * E + e] = s;
}
// out[e] = sum of the partials of column e, in fp64: a block holds 64
// columns x 4 slices of the chunks; each slice adds its chunks in order
// (requested 16 at a time), then the 4 slice sums are added in slice order.
__global__ __launch_bounds__(256) void colsum_final_kernel(const float* __restrict__ part,
                                                           int nchunk, int E,
                                                           float* __restrict__ out) {
  __shared__ double red[4][64];
  const int col = threadIdx.x & 63, sl = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + col;
  const int per = (nchunk + 3) / 4;
  const int c0 = sl * per, c1 = min(nchunk, c0 + per);
  double s = 0.0;
  if (e < E) {
    for (int cb = c0; cb < c1; cb += 16) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = cb + i < c1 ? part[(long long)(cb + i) * E + e] : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s += (double)v[i];
    }
  }
  red[sl][col] = s;
  __syncthreads();
  if (sl == 0 && e < E) out[e] = (float)(((red[0][col] + red[1][col]) + red[2][col]) + red[3][col]);
}

static int grid_for(long long n) {
  long long g = (n + 255) / 256;
  return (int)(g < 4096 ? (g < 1 ? 1 : g) : 4096);
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// workspace layout (bytes), forward and backward use it separately
struct RouterWs {
  size_t wg3s, wgb, part, dl3s, dlb, colpart, total;
};
static RouterWs router_ws_layout(int T, int H, int E) {
  RouterWs w = {};
  const size_t he = (size_t)H * E, te = (size_t)T * E;
  size_t o = 0;
  w.wg3s = o; o += align256(3 * he * 2);
  w.wgb = o; o += align256(he * 2);
  w.part = o;
  size_t part_bytes = (size_t)RT_SPLIT * (te > he ? te : he) * 4;
  o += align256(part_bytes);
  w.dl3s = o; o += align256(3 * te * 2);
  w.dlb = o; o += align256(te * 2);
  w.colpart = o; o += align256((size_t)((T + COLSUM_ROWS - 1) / COLSUM_ROWS) * E * 4);
  w.total = o;
  return w;
}

static int router_checks(const char* fn, int dt, int T, int H, int E) {
  MOE_TRY(moe_need_dt(dt, fn));
  MOE_TRY(moe_need_nonneg(T, fn, "T"));
  MOE_TRY(moe_need_mult64(H, fn, "H"));
  MOE_TRY(moe_need_ek(E, 1, fn));
  MOE_TRY(moe_need_elems(T, H, moe_dt_bytes(dt), fn, "x"));
  MOE_TRY(moe_need_elems(T, E, 4, fn, "logits"));
  MOE_TRY(moe_need_elems((long long)RT_SPLIT * T, E, 4, fn, "router partial sums"));
  return MOE_OK;
}

extern "C" size_t moe_router_workspace_bytes(int T, int H, int E, int dt) {
  if (T <= 0 || H <= 0 || E <= 0 || !mfma_path(dt, T, H, E)) return 0;
  return router_ws_layout(T, H, E).total;
}

extern "C" int moe_router_logits(const void* x, int dt, const float* wg, const float* bias, int T,
                                 int H, int E, float* logits, void* ws, size_t ws_bytes,
                                 moe_stream_t stream) {
  const char* fn = "moe_router_logits";
  MOE_TRY(router_checks(fn, dt, T, H, E));
  if (T == 0) return MOE_OK;
  MOE_TRY(moe_need_ptr(x, fn, "x"));
  MOE_TRY(moe_need_ptr(wg, fn, "wg", 4));
  MOE_TRY(moe_opt_ptr(bias, fn, "bias", 4));
  MOE_TRY(moe_need_ptr(logits, fn, "logits", 4));
  hipStream_t s = (hipStream_t)stream;
  if (mfma_path(dt, T, H, E)) {
    const size_t need = moe_router_workspace_bytes(T, H, E, dt);
    MOE_TRY(moe_need_ptr(ws, fn, "ws", 256));
    if (ws_bytes < need)
      return moe_fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    const RouterWs L = router_ws_layout(T, H, E);
    char* w = (char*)ws;
    bf16_t* wg3s = (bf16_t*)(w + L.wg3s);
    bf16_t* wgb = (bf16_t*)(w + L.wgb);
    float* part = (float*)(w + L.part);
    // the hi parts too: the backward can reuse this split (MOE_ROUTER_WG_SPLIT)
    hipLaunchKernelGGL(split_wg_kernel, dim3(grid_for((long long)H * E)), dim3(256), 0, s, wg, H, E,
                       wg3s, wgb);
    MOE_TRY(moe_check_launch(fn));
    MOE_TRY(moe_gmm_router_fwd(x, wg3s, part, T, H, E, RT_SPLIT, s));
    hipLaunchKernelGGL(reduce_slices_kernel, dim3(grid_for((long long)T * E)), dim3(256), 0, s,
                       (const float*)part, (long long)T * E, E, bias, logits);
    return moe_check_launch(fn);
  }
  if (dt == MOE_BF16)
    launch_router_gemm<bf16_t, float>(s, (const bf16_t*)x, H, 1, wg, E, 1, bias, T, E, H, logits, E);
  else
    launch_router_gemm<float, float>(s, (const float*)x, H, 1, wg, E, 1, bias, T, E, H, logits, E);
  return moe_check_launch(fn);
}

extern "C" int moe_router_logits_bwd(const float* dlogits, const void* x, int dt, const float* wg,
                                     int T, int H, int E, void* dx, float* dwg, float* dbias,
                                     int flags, void* ws, size_t ws_bytes, moe_stream_t stream) {
  const char* fn = "moe_router_logits_bwd";
  MOE_TRY(router_checks(fn, dt, T, H, E));
  if (flags & ~MOE_ROUTER_WG_SPLIT)
    return moe_fail(MOE_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
  MOE_TRY(moe_need_ptr(dwg, fn, "dwg", 4));
  MOE_TRY(moe_opt_ptr(dbias, fn, "dbias", 4));
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {
    // no tokens: the weight gradients are zero
    hipLaunchKernelGGL((router_gemm_kernel<float, float>), dim3((E + RT_BN - 1) / RT_BN, (H + RT_BM - 1) / RT_BM),
                       dim3(256), 0, s, (const float*)nullptr, 0LL, 0LL, (const float*)nullptr, 0LL,
                       0LL, (const float*)nullptr, H, E, 0, dwg, (long long)E);
    if (dbias)
      hipLaunchKernelGGL(colsum_final_kernel, dim3((E + 63) / 64), dim3(256), 0, s,
                         (const float*)nullptr, 0, E, dbias);
    return moe_check_launch(fn);
  }
  MOE_TRY(moe_need_ptr(dlogits, fn, "dlogits", 4));
  MOE_TRY(moe_need_ptr(x, fn, "x"));
  MOE_TRY(moe_need_ptr(wg, fn, "wg", 4));
  MOE_TRY(moe_need_ptr(dx, fn, "dx"));
  const bool mfma = mfma_path(dt, T, H, E);
  RouterWs L = router_ws_layout(T, H, E);
  if (mfma || dbias) {
    const size_t need = mfma ? L.total : 0;
    if (mfma) {
      MOE_TRY(moe_need_ptr(ws, fn, "ws", 256));
      if (ws_bytes < need)
        return moe_fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes,
                        need);
    }
  }
  const int nchunk = (T + COLSUM_ROWS - 1) / COLSUM_ROWS;
  if (mfma) {
    char* w = (char*)ws;
    bf16_t* wg3s = (bf16_t*)(w + L.wg3s);
    bf16_t* wgb = (bf16_t*)(w + L.wgb);
    float* part = (float*)(w + L.part);
    bf16_t* dl3s = (bf16_t*)(w + L.dl3s);
    bf16_t* dlb = (bf16_t*)(w + L.dlb);
    if (!(flags & MOE_ROUTER_WG_SPLIT)) {
      hipLaunchKernelGGL(split_wg_kernel, dim3(grid_for((long long)H * E)), dim3(256), 0, s, wg, H,
                         E, wg3s, wgb);
      MOE_TRY(moe_check_launch(fn));
    }
    hipLaunchKernelGGL(split_dl_kernel, dim3(grid_for((long long)T * E)), dim3(256), 0, s, dlogits,
                       T, E, dl3s, dlb);
    MOE_TRY(moe_check_launch(fn));
    MOE_TRY(moe_gmm_router_dx(dlb, wgb, dx, T, H, E, s));
    MOE_TRY(moe_gmm_router_dwg(x, dl3s, part, T, H, E, RT_SPLIT, s));
    hipLaunchKernelGGL(reduce_slices_kernel, dim3(grid_for((long long)H * E)), dim3(256), 0, s,
                       (const float*)part, (long long)H * E, E, (const float*)nullptr, dwg);
    MOE_TRY(moe_check_launch(fn));
    if (dbias) {
      float* colpart = (float*)(w + L.colpart);
      hipLaunchKernelGGL(colsum_part_kernel, dim3(nchunk, (E + 255) / 256), dim3(256), 0, s,
                         dlogits, T, E, colpart);
      hipLaunchKernelGGL(colsum_final_kernel, dim3((E + 63) / 64), dim3(256), 0, s,
                         (const float*)colpart, nchunk, E, dbias);
      MOE_TRY(moe_check_launch(fn));
    }
    return MOE_OK;
  }
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
    // small shapes: one fixed-order column sum per expert
    hipLaunchKernelGGL(colsum_kernel, dim3((E + MOE_WAVE - 1) / MOE_WAVE), dim3(1024), 0, s,
                       dlogits, T, E, dbias);
    MOE_TRY(moe_check_launch(fn));
  }
  return MOE_OK;
}
