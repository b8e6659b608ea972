// Permute (reorder tokens into per-expert groups), its backward, and the
// unpermute + gate-weighted combine with its backward ([MoE-ops] VectorSort,
// Fig. 3; [MoE-ops] Host-Device section, Fig. 4: the per-expert counts are
// produced and consumed on the device, never read back by the host).
//
// Stable rank without atomics: tokens are cut into chunks of PERM_CHUNK; one
// wavefront per chunk walks its tokens in order and counts, per expert, the
// earlier tokens of the chunk (the local rank).  A column scan over chunks
// gives each chunk's base inside every expert group and the counts; a scan
// over experts gives the group offsets.  The row of pair (t,j) is then
// offsets[e] + chunk base + local rank, unique and in token order.
//
// The row moves are token-centric: one workgroup per token reads the token's
// row once with 16-byte lanes and writes (or gathers) its k rows.
#include "validate.hpp"

#define PERM_CHUNK 32      // tokens per rank chunk
#define ROW_THREADS 256    // threads of a row-moving workgroup
#define ROW_MAXC 8         // 16-byte chunks per thread kept in registers

static inline long long perm_chunks(int T) { return (T + PERM_CHUNK - 1) / PERM_CHUNK; }

// ---------------------------------------------------------------- rank

__global__ __launch_bounds__(MOE_WAVE) void permute_rank_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int32_t* __restrict__ local_rank,
    int32_t* __restrict__ hist) {
  __shared__ int cnt[MOE_MAX_E];
  __shared__ int ids[PERM_CHUNK * 64];
  const int lane = threadIdx.x;
  const int c = blockIdx.x;
  const int t0 = c * PERM_CHUNK;
  const int nt = min(PERM_CHUNK, T - t0);
  for (int e = lane; e < E; e += MOE_WAVE) cnt[e] = 0;
  // stage the chunk's expert ids (nt*k of them) through LDS in pieces of
  // PERM_CHUNK*64 values
  const long long base = (long long)t0 * k;
  const int total = nt * k;
  const int piece = ((PERM_CHUNK * 64) / k) * k;  // whole tokens per piece (k <= 1024)
  for (int p0 = 0; p0 < total; p0 += piece) {
    const int pn = min(piece, total - p0);
    for (int i = lane; i < pn; i += MOE_WAVE) {
      int e = idx[base + p0 + i];
      ids[i] = (e >= 0 && e < E) ? e : 0;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // walk the pairs in order; the k experts of one token are distinct, so
    // the lanes of one step touch distinct counters
    for (int q = 0; q < pn; q += k) {
      for (int j = lane; j < k && q + j < pn; j += MOE_WAVE) {
        int e = ids[q + j];
        int r = cnt[e];
        cnt[e] = r + 1;
        local_rank[base + p0 + q + j] = r;
      }
      __builtin_amdgcn_wave_barrier();
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
  }
  for (int e = lane; e < E; e += MOE_WAVE) hist[(long long)c * E + e] = cnt[e];
}

// Column scan over chunks: hist[c][e] <- sum_{c' < c} hist[c'][e];
// counts[e] <- sum_c hist[c][e].  Block: 64 experts x 16 chunk slices.
#define SCAN_SLICES 16
__global__ __launch_bounds__(MOE_WAVE * SCAN_SLICES) void permute_colscan_kernel(
    int32_t* __restrict__ hist, int nchunks, int E, int32_t* __restrict__ counts) {
  __shared__ int part[SCAN_SLICES][MOE_WAVE];
  const int lane = threadIdx.x % MOE_WAVE;
  const int s = threadIdx.x / MOE_WAVE;
  const int e = blockIdx.x * MOE_WAVE + lane;
  const int per = (nchunks + SCAN_SLICES - 1) / SCAN_SLICES;
  const int c0 = s * per, c1 = min(nchunks, c0 + per);
  int sum = 0;
  if (e < E)
    for (int c = c0; c < c1; ++c) sum += hist[(long long)c * E + e];
  part[s][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int i = 0; i < s; ++i) run += part[i][lane];
  if (e < E) {
    for (int c = c0; c < c1; ++c) {
      long long o = (long long)c * E + e;
      int v = hist[o];
      hist[o] = run;
      run += v;
    }
    if (s == SCAN_SLICES - 1) counts[e] = run;
  }
}

// offsets = exclusive scan of counts, offsets[E] = total.  One block of 1024.
__global__ __launch_bounds__(1024) void permute_offsets_kernel(const int32_t* __restrict__ counts,
                                                               int E, int32_t* __restrict__ offsets) {
  __shared__ int buf[1024];
  const int i = threadIdx.x;
  int v = i < E ? counts[i] : 0;
  buf[i] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int add = i >= o ? buf[i - o] : 0;
    __syncthreads();
    buf[i] += add;
    __syncthreads();
  }
  if (i < E) offsets[i] = buf[i] - v;
  if (i == E - 1) offsets[E] = buf[i];
}

__global__ __launch_bounds__(1024) void permute_zero_kernel(int32_t* counts, int32_t* offsets,
                                                            int E) {
  for (int i = threadIdx.x; i <= E; i += 1024) {
    if (i < E) counts[i] = 0;
    offsets[i] = 0;
  }
}

// ---------------------------------------------------------------- load statistics

// Fixed-order sum over the block (shuffle tree per wave, then the 16 wave
// sums in order): bitwise the same on every run.
__device__ __forceinline__ double stats_block_sum(double v, double* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  __syncthreads();                       // red is free again
  if (threadIdx.x % MOE_WAVE == 0) red[threadIdx.x / MOE_WAVE] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < 1024 / MOE_WAVE; ++w) s += red[w];
  return s;
}

// Per-expert load, cv of the loads, EP-group counts and their cv from one
// step's counts (moe_load_stats).  One block of 1024 threads, thread i owns
// expert i and, for i < E / epg, EP group i.  fp64 inside.
__global__ __launch_bounds__(1024) void load_stats_kernel(const int32_t* __restrict__ counts,
                                                          int E, int epg,
                                                          float* __restrict__ load,
                                                          float* __restrict__ cv,
                                                          int32_t* __restrict__ group_counts) {
  __shared__ int cnt[1024];
  __shared__ double red[1024 / MOE_WAVE];
  const int i = threadIdx.x;
  const int c = i < E ? counts[i] : 0;
  cnt[i] = c;
  // counts are integers below 2^31 and at most 1024 of them: the fp64 sum is exact
  const double total = stats_block_sum((double)c, red);
  const double mean = total / E;
  const double d = i < E ? (double)c - mean : 0.0;
  const double var = stats_block_sum(d * d, red) / E;
  if (load != nullptr && i < E) load[i] = total > 0.0 ? (float)((double)c / total) : 0.f;
  const int G = E / epg;
  double gs = 0.0;
  if (i < G) {
    for (int j = 0; j < epg; ++j) gs += (double)cnt[i * epg + j];
    if (group_counts != nullptr) group_counts[i] = (int32_t)gs;
  }
  const double gmean = total / G;
  const double gd = i < G ? gs - gmean : 0.0;
  const double gvar = stats_block_sum(gd * gd, red) / G;
  if (cv != nullptr && i == 0) {
    cv[0] = total > 0.0 ? (float)(sqrt(var) / mean) : 0.f;
    cv[1] = total > 0.0 ? (float)(sqrt(gvar) / gmean) : 0.f;
  }
}

// ---------------------------------------------------------------- scatter

template <int ESZ>
__global__ __launch_bounds__(ROW_THREADS) void permute_scatter_kernel(
    const void* __restrict__ x, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ hist, int T, int H, int E,
    int k, void* __restrict__ xp, int32_t* __restrict__ row_id_map,
    int32_t* __restrict__ src_token) {
  __shared__ int rows[MOE_MAX_E];
  const int t = blockIdx.x;
  const long long R = (long long)T * k;
  const int c = t / PERM_CHUNK;
  for (int j = threadIdx.x; j < k; j += ROW_THREADS) {
    long long p = (long long)t * k + j;
    int e = idx[p];
    e = (e >= 0 && e < E) ? e : 0;
    long long row = (long long)offsets[e] + hist[(long long)c * E + e] + row_id_map[p];
    row = row < 0 ? 0 : (row >= R ? R - 1 : row);
    row_id_map[p] = (int)row;
    src_token[row] = t;
    rows[j] = (int)row;
  }
  __syncthreads();
  const uint32_t row_bytes = (uint32_t)H * ESZ;
  const int nchunk = row_bytes / 16;
  __amdgpu_buffer_rsrc_t src = make_rsrc((const char*)x + (long long)t * row_bytes, row_bytes);
  __amdgpu_buffer_rsrc_t dst = make_rsrc(xp, clamp_bytes(R * row_bytes));
  for (int q0 = 0; q0 < nchunk; q0 += ROW_THREADS * ROW_MAXC) {
    u32x4 v[ROW_MAXC];
#pragma unroll
    for (int i = 0; i < ROW_MAXC; ++i) {
      int q = q0 + i * ROW_THREADS + threadIdx.x;
      v[i] = buf_load16_nt(src, (uint32_t)q * 16u);
    }
    for (int j = 0; j < k; ++j) {
      const uint32_t rb = (uint32_t)rows[j] * row_bytes;
#pragma unroll
      for (int i = 0; i < ROW_MAXC; ++i) {
        int q = q0 + i * ROW_THREADS + threadIdx.x;
        if (q < nchunk) buf_store16(dst, rb + (uint32_t)q * 16u, v[i]);
      }
    }
  }
}

// Row map and source tokens only (no row copy): one thread per (t, j).
__global__ __launch_bounds__(256) void permute_maps_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ hist, int T, int E, int k, int32_t* __restrict__ row_id_map,
    int32_t* __restrict__ src_token) {
  const long long R = (long long)T * k;
  const long long p = (long long)blockIdx.x * 256 + threadIdx.x;
  if (p >= R) return;
  const int t = (int)(p / k);
  const int c = t / PERM_CHUNK;
  int e = idx[p];
  e = (e >= 0 && e < E) ? e : 0;
  long long row = (long long)offsets[e] + hist[(long long)c * E + e] + row_id_map[p];
  row = row < 0 ? 0 : (row >= R ? R - 1 : row);
  row_id_map[p] = (int)row;
  src_token[row] = t;
}

// ---------------------------------------------------------------- gathers
// The gathers below keep ROW_JB rows x ROW_QB chunks of loads in flight per
// thread (requested together, then added in row order), so a token's k row
// reads overlap instead of paying one HBM latency each.
#define ROW_JB 8   // rows requested together
#define ROW_QB 4   // 16-byte chunks per thread per pass

// chunk q of row r (zero for q past the row); every row the gathers read is
// read once, so the loads stream past the caches
__device__ __forceinline__ u32x4 row_chunk(const __amdgpu_buffer_rsrc_t& rs, uint32_t rb, int q,
                                           int nchunk) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (q < nchunk) v = buf_load16_nt(rs, rb + (uint32_t)q * 16u);
  return v;
}

// ---------------------------------------------------------------- permute bwd
// dx[t] = sum_j dxp[row(t,j)] + add0[t] + add1[t]   (fp32 sums, j ascending)

template <typename T>
__global__ __launch_bounds__(ROW_THREADS) void permute_bwd_kernel(
    const T* __restrict__ dxp, const int32_t* __restrict__ row_id_map, int Tn, int H, int k,
    const T* __restrict__ add0, const T* __restrict__ add1, T* __restrict__ dx) {
  constexpr int VEC = Elem<T>::VEC;
  __shared__ int rows[MOE_MAX_E];
  const int t = blockIdx.x;
  const long long R = (long long)Tn * k;
  for (int j = threadIdx.x; j < k; j += ROW_THREADS) {
    long long row = row_id_map[(long long)t * k + j];
    rows[j] = (int)(row < 0 ? 0 : (row >= R ? R - 1 : row));
  }
  __syncthreads();
  const uint32_t row_bytes = (uint32_t)H * sizeof(T);
  const int nchunk = row_bytes / 16;
  __amdgpu_buffer_rsrc_t src = make_rsrc(dxp, clamp_bytes(R * row_bytes));
  __amdgpu_buffer_rsrc_t out = make_rsrc((char*)dx + (long long)t * row_bytes, row_bytes);
  __amdgpu_buffer_rsrc_t a0 = make_rsrc(add0 ? (const char*)add0 + (long long)t * row_bytes : nullptr,
                                        add0 ? row_bytes : 0);
  __amdgpu_buffer_rsrc_t a1 = make_rsrc(add1 ? (const char*)add1 + (long long)t * row_bytes : nullptr,
                                        add1 ? row_bytes : 0);
  for (int q0 = threadIdx.x; q0 < nchunk; q0 += ROW_QB * ROW_THREADS) {
    float acc[ROW_QB][VEC], tmp[VEC];
#pragma unroll
    for (int u = 0; u < ROW_QB; ++u)
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[u][i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += ROW_JB) {
      u32x4 v[ROW_JB][ROW_QB];
#pragma unroll
      for (int jj = 0; jj < ROW_JB; ++jj)
        if (j0 + jj < k) {
          const uint32_t rb = (uint32_t)rows[j0 + jj] * row_bytes;
#pragma unroll
          for (int u = 0; u < ROW_QB; ++u) v[jj][u] = row_chunk(src, rb, q0 + u * ROW_THREADS, nchunk);
        }
#pragma unroll
      for (int jj = 0; jj < ROW_JB; ++jj)
        if (j0 + jj < k) {
#pragma unroll
          for (int u = 0; u < ROW_QB; ++u) {
            unpack16(v[jj][u], tmp, T());
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[u][i] += tmp[i];
          }
        }
    }
    u32x4 e0[ROW_QB], e1[ROW_QB];
#pragma unroll
    for (int u = 0; u < ROW_QB; ++u) {
      e0[u] = add0 ? row_chunk(a0, 0, q0 + u * ROW_THREADS, nchunk) : u32x4{0u, 0u, 0u, 0u};
      e1[u] = add1 ? row_chunk(a1, 0, q0 + u * ROW_THREADS, nchunk) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < ROW_QB; ++u) {
      const int q = q0 + u * ROW_THREADS;
      if (add0) {
        unpack16(e0[u], tmp, T());
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[u][i] += tmp[i];
      }
      if (add1) {
        unpack16(e1[u], tmp, T());
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[u][i] += tmp[i];
      }
      if (q < nchunk) buf_store16(out, (uint32_t)q * 16u, pack16(acc[u], T()));
    }
  }
}

// ---------------------------------------------------------------- combine
// y[t] = ys[t] + sum_j gate[t,j] yp[row(t,j)]   (fp32, j ascending)

template <typename T>
__global__ __launch_bounds__(ROW_THREADS) void combine_kernel(
    const T* __restrict__ yp, const int32_t* __restrict__ row_id_map,
    const float* __restrict__ gate, const T* __restrict__ ys, int Tn, int H, int k,
    T* __restrict__ y) {
  constexpr int VEC = Elem<T>::VEC;
  __shared__ int rows[MOE_MAX_E];
  __shared__ float gates[MOE_MAX_E];
  const int t = blockIdx.x;
  const long long R = (long long)Tn * k;
  for (int j = threadIdx.x; j < k; j += ROW_THREADS) {
    long long row = row_id_map[(long long)t * k + j];
    rows[j] = (int)(row < 0 ? 0 : (row >= R ? R - 1 : row));
    gates[j] = gate[(long long)t * k + j];
  }
  __syncthreads();
  const uint32_t row_bytes = (uint32_t)H * sizeof(T);
  const int nchunk = row_bytes / 16;
  __amdgpu_buffer_rsrc_t src = make_rsrc(yp, clamp_bytes(R * row_bytes));
  __amdgpu_buffer_rsrc_t out = make_rsrc((char*)y + (long long)t * row_bytes, row_bytes);
  __amdgpu_buffer_rsrc_t sh = make_rsrc(ys ? (const char*)ys + (long long)t * row_bytes : nullptr,
                                        ys ? row_bytes : 0);
  for (int q0 = threadIdx.x; q0 < nchunk; q0 += ROW_QB * ROW_THREADS) {
    float acc[ROW_QB][VEC], tmp[VEC];
#pragma unroll
    for (int u = 0; u < ROW_QB; ++u) {
      if (ys) {
        unpack16(row_chunk(sh, 0, q0 + u * ROW_THREADS, nchunk), acc[u], T());
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[u][i] = 0.f;
      }
    }
    for (int j0 = 0; j0 < k; j0 += ROW_JB) {
      u32x4 v[ROW_JB][ROW_QB];
#pragma unroll
      for (int jj = 0; jj < ROW_JB; ++jj)
        if (j0 + jj < k) {
          const uint32_t rb = (uint32_t)rows[j0 + jj] * row_bytes;
#pragma unroll
          for (int u = 0; u < ROW_QB; ++u) v[jj][u] = row_chunk(src, rb, q0 + u * ROW_THREADS, nchunk);
        }
#pragma unroll
      for (int jj = 0; jj < ROW_JB; ++jj)
        if (j0 + jj < k) {
          const float g = gates[j0 + jj];
#pragma unroll
          for (int u = 0; u < ROW_QB; ++u) {
            unpack16(v[jj][u], tmp, T());
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[u][i] += g * tmp[i];
          }
        }
    }
#pragma unroll
    for (int u = 0; u < ROW_QB; ++u) {
      const int q = q0 + u * ROW_THREADS;
      if (q < nchunk) buf_store16(out, (uint32_t)q * 16u, pack16(acc[u], T()));
    }
  }
}

// dyp[row(t,j)] = gate[t,j] dy[t];  dgate[t,j] = <dy[t], yp[row(t,j)]>
// (per thread fp32 partial dots over its chunks, then a fixed-order
// reduction: wave sums, then the waves in order)
template <typename T>
__global__ __launch_bounds__(ROW_THREADS) void combine_bwd_kernel(
    const T* __restrict__ dy, const T* __restrict__ yp, const int32_t* __restrict__ row_id_map,
    const float* __restrict__ gate, int Tn, int H, int k, T* __restrict__ dyp,
    float* __restrict__ dgate) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int NW = ROW_THREADS / MOE_WAVE;
  __shared__ int rows[MOE_MAX_E];
  __shared__ float gates[MOE_MAX_E];
  __shared__ float red[ROW_JB][NW];
  const int t = blockIdx.x;
  const long long R = (long long)Tn * k;
  for (int j = threadIdx.x; j < k; j += ROW_THREADS) {
    long long row = row_id_map[(long long)t * k + j];
    rows[j] = (int)(row < 0 ? 0 : (row >= R ? R - 1 : row));
    gates[j] = gate[(long long)t * k + j];
  }
  __syncthreads();
  const uint32_t row_bytes = (uint32_t)H * sizeof(T);
  const int nchunk = row_bytes / 16;
  __amdgpu_buffer_rsrc_t din = make_rsrc((const char*)dy + (long long)t * row_bytes, row_bytes);
  __amdgpu_buffer_rsrc_t ypr = make_rsrc(yp, clamp_bytes(R * row_bytes));
  __amdgpu_buffer_rsrc_t dst = make_rsrc(dyp, clamp_bytes(R * row_bytes));
  const int lane = threadIdx.x % MOE_WAVE, w = threadIdx.x / MOE_WAVE;
  // the token's dy row stays in registers (ROW_MAXC chunks per thread)
  u32x4 draw[ROW_MAXC];
#pragma unroll
  for (int c = 0; c < ROW_MAXC; ++c)
    draw[c] = row_chunk(din, 0, threadIdx.x + c * ROW_THREADS, nchunk);
  for (int j0 = 0; j0 < k; j0 += ROW_JB) {
    float part[ROW_JB];
#pragma unroll
    for (int jj = 0; jj < ROW_JB; ++jj) part[jj] = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < ROW_MAXC; c0 += ROW_QB) {
      if (c0 * ROW_THREADS >= nchunk) break;   // uniform
      u32x4 v[ROW_JB][ROW_QB];
#pragma unroll
      for (int jj = 0; jj < ROW_JB; ++jj)
        if (j0 + jj < k) {
          const uint32_t rb = (uint32_t)rows[j0 + jj] * row_bytes;
#pragma unroll
          for (int u = 0; u < ROW_QB; ++u)
            v[jj][u] = row_chunk(ypr, rb, threadIdx.x + (c0 + u) * ROW_THREADS, nchunk);
        }
#pragma unroll
      for (int jj = 0; jj < ROW_JB; ++jj)
        if (j0 + jj < k) {
          const uint32_t rb = (uint32_t)rows[j0 + jj] * row_bytes;
          const float g = gates[j0 + jj];
#pragma unroll
          for (int u = 0; u < ROW_QB; ++u) {
            const int q = threadIdx.x + (c0 + u) * ROW_THREADS;
            float d[VEC], tmp[VEC], o[VEC];
            unpack16(draw[c0 + u], d, T());
            unpack16(v[jj][u], tmp, T());
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
              part[jj] += d[i] * tmp[i];
              o[i] = g * d[i];
            }
            if (q < nchunk) buf_store16(dst, rb + (uint32_t)q * 16u, pack16(o, T()));
          }
        }
    }
#pragma unroll
    for (int jj = 0; jj < ROW_JB; ++jj) {
      const float ps = wave_sum(part[jj]);
      if (lane == 0) red[jj][w] = ps;
    }
    __syncthreads();
    if (threadIdx.x < ROW_JB && j0 + (int)threadIdx.x < k) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) sum += red[threadIdx.x][i];
      dgate[(long long)t * k + j0 + threadIdx.x] = sum;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- C ABI

static int row_checks(const char* fn, int dt, int T, int H, int k) {
  MOE_TRY(moe_need_dt(dt, fn));
  MOE_TRY(moe_need_nonneg(T, fn, "T"));
  MOE_TRY(moe_need_mult64(H, fn, "H"));
  if (k < 1 || k > MOE_MAX_E)
    return moe_fail(MOE_ERR_UNSUPPORTED, "%s: k = %d outside [1, %d]", fn, k, MOE_MAX_E);
  const long long row_bytes = (long long)H * moe_dt_bytes(dt);
  if (row_bytes > 16LL * ROW_THREADS * ROW_MAXC)
    return moe_fail(MOE_ERR_UNSUPPORTED, "%s: a row of H = %d elements exceeds %d bytes", fn, H,
                    16 * ROW_THREADS * ROW_MAXC);
  MOE_TRY(moe_need_elems((long long)T * k, H, moe_dt_bytes(dt), fn, "permuted rows"));
  return MOE_OK;
}

extern "C" size_t moe_permute_workspace_bytes(int T, int E, int k) {
  (void)k;
  if (T <= 0 || E <= 0) return 0;
  return (size_t)perm_chunks(T) * (size_t)E * sizeof(int32_t);
}

extern "C" int moe_permute(const void* x, int dt, const int32_t* idx, int T, int H, int E, int k,
                           void* xp, int32_t* counts, int32_t* offsets, int32_t* row_id_map,
                           int32_t* src_token, void* ws, size_t ws_bytes, moe_stream_t stream) {
  const char* fn = "moe_permute";
  MOE_TRY(row_checks(fn, dt, T, H, k));
  MOE_TRY(moe_need_ek(E, k, fn));
  MOE_TRY(moe_need_ptr(counts, fn, "counts", 4));
  MOE_TRY(moe_need_ptr(offsets, fn, "offsets", 4));
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {
    // empty input: every group is empty (a fill kernel, not a memset node)
    hipLaunchKernelGGL(permute_zero_kernel, dim3(1), dim3(1024), 0, s, counts, offsets, E);
    return moe_check_launch("moe_permute(empty)");
  }
  MOE_TRY(xp ? moe_need_ptr(x, fn, "x") : moe_opt_ptr(x, fn, "x"));
  MOE_TRY(moe_need_ptr(idx, fn, "idx", 4));
  MOE_TRY(moe_opt_ptr(xp, fn, "xp"));
  MOE_TRY(moe_need_ptr(row_id_map, fn, "row_id_map", 4));
  MOE_TRY(moe_need_ptr(src_token, fn, "src_token", 4));
  MOE_TRY(moe_need_ptr(ws, fn, "ws", 4));
  if (ws_bytes < moe_permute_workspace_bytes(T, E, k))
    return moe_fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes,
                    moe_permute_workspace_bytes(T, E, k));
  const int nchunks = (int)perm_chunks(T);
  int32_t* hist = (int32_t*)ws;
  hipLaunchKernelGGL(permute_rank_kernel, dim3(nchunks), dim3(MOE_WAVE), 0, s, idx, T, E, k,
                     row_id_map, hist);
  MOE_TRY(moe_check_launch("moe_permute(rank)"));
  hipLaunchKernelGGL(permute_colscan_kernel, dim3((E + MOE_WAVE - 1) / MOE_WAVE),
                     dim3(MOE_WAVE * SCAN_SLICES), 0, s, hist, nchunks, E, counts);
  MOE_TRY(moe_check_launch("moe_permute(scan)"));
  hipLaunchKernelGGL(permute_offsets_kernel, dim3(1), dim3(1024), 0, s, counts, E, offsets);
  MOE_TRY(moe_check_launch("moe_permute(offsets)"));
  if (xp == nullptr) {
    const long long R = (long long)T * k;
    hipLaunchKernelGGL(permute_maps_kernel, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, s,
                       idx, offsets, hist, T, E, k, row_id_map, src_token);
    return moe_check_launch("moe_permute(maps)");
  }
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(permute_scatter_kernel<2>, dim3(T), dim3(ROW_THREADS), 0, s, x, idx,
                       offsets, hist, T, H, E, k, xp, row_id_map, src_token);
  else
    hipLaunchKernelGGL(permute_scatter_kernel<4>, dim3(T), dim3(ROW_THREADS), 0, s, x, idx,
                       offsets, hist, T, H, E, k, xp, row_id_map, src_token);
  return moe_check_launch("moe_permute(scatter)");
}

extern "C" int moe_load_stats(const int32_t* counts, int E, int experts_per_group, float* load,
                              float* cv, int32_t* group_counts, moe_stream_t stream) {
  const char* fn = "moe_load_stats";
  if (E < 1 || E > MOE_MAX_E)
    return moe_fail(MOE_ERR_UNSUPPORTED, "%s: E = %d outside [1, %d]", fn, E, MOE_MAX_E);
  if (experts_per_group < 1 || E % experts_per_group != 0)
    return moe_fail(MOE_ERR_INVALID_ARG, "%s: experts_per_group = %d does not divide E = %d", fn,
                    experts_per_group, E);
  MOE_TRY(moe_need_ptr(counts, fn, "counts", 4));
  MOE_TRY(moe_opt_ptr(load, fn, "load", 4));
  MOE_TRY(moe_opt_ptr(cv, fn, "cv", 4));
  MOE_TRY(moe_opt_ptr(group_counts, fn, "group_counts", 4));
  hipLaunchKernelGGL(load_stats_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, counts, E,
                     experts_per_group, load, cv, group_counts);
  return moe_check_launch(fn);
}

extern "C" int moe_permute_bwd(const void* dxp, const int32_t* row_id_map, int dt, int T, int H,
                               int k, const void* add0, const void* add1, void* dx,
                               moe_stream_t stream) {
  const char* fn = "moe_permute_bwd";
  MOE_TRY(row_checks(fn, dt, T, H, k));
  if (T == 0) return MOE_OK;
  MOE_TRY(moe_need_ptr(dxp, fn, "dxp"));
  MOE_TRY(moe_need_ptr(row_id_map, fn, "row_id_map", 4));
  MOE_TRY(moe_need_ptr(dx, fn, "dx"));
  MOE_TRY(moe_opt_ptr(add0, fn, "add0"));
  MOE_TRY(moe_opt_ptr(add1, fn, "add1"));
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(permute_bwd_kernel<bf16_t>, dim3(T), dim3(ROW_THREADS), 0, s,
                       (const bf16_t*)dxp, row_id_map, T, H, k, (const bf16_t*)add0,
                       (const bf16_t*)add1, (bf16_t*)dx);
  else
    hipLaunchKernelGGL(permute_bwd_kernel<float>, dim3(T), dim3(ROW_THREADS), 0, s,
                       (const float*)dxp, row_id_map, T, H, k, (const float*)add0,
                       (const float*)add1, (float*)dx);
  return moe_check_launch(fn);
}

extern "C" int moe_unpermute_combine(const void* yp, const int32_t* row_id_map, const float* gate,
                                     const void* y_shared, int dt, int T, int H, int k, void* y,
                                     moe_stream_t stream) {
  const char* fn = "moe_unpermute_combine";
  MOE_TRY(row_checks(fn, dt, T, H, k));
  if (T == 0) return MOE_OK;
  MOE_TRY(moe_need_ptr(yp, fn, "yp"));
  MOE_TRY(moe_need_ptr(row_id_map, fn, "row_id_map", 4));
  MOE_TRY(moe_need_ptr(gate, fn, "gate", 4));
  MOE_TRY(moe_opt_ptr(y_shared, fn, "y_shared"));
  MOE_TRY(moe_need_ptr(y, fn, "y"));
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(T), dim3(ROW_THREADS), 0, s,
                       (const bf16_t*)yp, row_id_map, gate, (const bf16_t*)y_shared, T, H, k,
                       (bf16_t*)y);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(T), dim3(ROW_THREADS), 0, s, (const float*)yp,
                       row_id_map, gate, (const float*)y_shared, T, H, k, (float*)y);
  return moe_check_launch(fn);
}

extern "C" int moe_unpermute_combine_bwd(const void* dy, const void* yp, const int32_t* row_id_map,
                                         const float* gate, int dt, int T, int H, int k, void* dyp,
                                         float* dgate, moe_stream_t stream) {
  const char* fn = "moe_unpermute_combine_bwd";
  MOE_TRY(row_checks(fn, dt, T, H, k));
  if (T == 0) return MOE_OK;
  MOE_TRY(moe_need_ptr(dy, fn, "dy"));
  MOE_TRY(moe_need_ptr(yp, fn, "yp"));
  MOE_TRY(moe_need_ptr(row_id_map, fn, "row_id_map", 4));
  MOE_TRY(moe_need_ptr(gate, fn, "gate", 4));
  MOE_TRY(moe_need_ptr(dyp, fn, "dyp"));
  MOE_TRY(moe_need_ptr(dgate, fn, "dgate", 4));
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(combine_bwd_kernel<bf16_t>, dim3(T), dim3(ROW_THREADS), 0, s,
                       (const bf16_t*)dy, (const bf16_t*)yp, row_id_map, gate, T, H, k,
                       (bf16_t*)dyp, dgate);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<float>, dim3(T), dim3(ROW_THREADS), 0, s,
                       (const float*)dy, (const float*)yp, row_id_map, gate, T, H, k,
                       (float*)dyp, dgate);
  return moe_check_launch(fn);
}
