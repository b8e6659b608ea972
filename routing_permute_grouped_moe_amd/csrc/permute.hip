// Permute (reorder tokens into per-expert groups), its backward, and the
// unpermute + gate-weighted combine with its backward ([MoE-ops] VectorSort,
// Fig. 3; [MoE-ops] Host-Device section, Fig. 4: the per-expert counts are
// produced and consumed on the device, never read back by the host).
//
// Stable rank without atomics: the T*k (token, slot) pairs, in pair order,
// are cut into blocks of RANK_BLOCK_PAIRS.  Inside a block every wavefront
// ranks 64 pairs at a time: the lanes holding the same expert find each other
// with one ballot per bit of the expert id, so a pair's rank among the step's
// pairs of its expert is the number of lower lanes that match, and the
// wave's per-expert counter in LDS gives the earlier steps' pairs.  The
// waves' counters are then scanned in wave order, which makes the rank
// relative to the block.  One more workgroup scans the blocks' counts per
// expert (each block's base inside every expert group, and the counts) and
// the counts over experts (the group offsets).  The row of pair (t,j) is
// offsets[e] + block base + rank in the block: unique and in token order.
//
// The row moves are token-centric: one workgroup per token reads the token's
// row once with 16-byte lanes and writes (or gathers) its k rows.
#include <mutex>

#include "validate.hpp"

#define RANK_WAVES 16      // wavefronts of a rank workgroup
#define RANK_STEPS 4       // 64-pair steps per wavefront
#define RANK_WAVE_PAIRS (MOE_WAVE * RANK_STEPS)
#define RANK_BLOCK_PAIRS (RANK_WAVES * RANK_WAVE_PAIRS)   // 4096 pairs per block
#define ROW_THREADS 256    // threads of a row-moving workgroup
#define ROW_MAXC 8         // 16-byte chunks per thread kept in registers

static inline long long rank_blocks(int T, int k) {
  return ((long long)T * k + RANK_BLOCK_PAIRS - 1) / RANK_BLOCK_PAIRS;
}

// Byte offset of a row that is not there (a dropped pair, or a row index
// outside [0, R)): every permuted-row buffer's descriptor stops at or before
// ROW_DROP bytes, so loads from it read zero and stores to it are discarded.
#define ROW_DROP 0xFFFF0000u
__device__ __forceinline__ uint32_t row_off(long long row, long long R, uint32_t row_bytes) {
  return (row >= 0 && row < R) ? (uint32_t)row * row_bytes : ROW_DROP;
}
__host__ __device__ __forceinline__ uint32_t rows_bytes(long long R, uint32_t row_bytes) {
  const long long b = R * (long long)row_bytes;
  return b <= 0 ? 0u : (b >= (long long)ROW_DROP ? ROW_DROP : (uint32_t)b);
}

// ---------------------------------------------------------------- rank

// local_rank[p] <- rank of pair p among the pairs of its expert in its block
// (pair order); hist[b][e] <- pairs of expert e in block b.  Dynamic LDS:
// RANK_WAVES * E counters.  ebits = bits of the largest expert id.
__global__ __launch_bounds__(MOE_WAVE * RANK_WAVES) void permute_rank_kernel(
    const int32_t* __restrict__ idx, long long P, int E, int ebits,
    int32_t* __restrict__ local_rank, int32_t* __restrict__ hist) {
  extern __shared__ int wcnt[];   // [RANK_WAVES][E]
  const int lane = threadIdx.x % MOE_WAVE, wave = threadIdx.x / MOE_WAVE;
  for (int i = threadIdx.x; i < RANK_WAVES * E; i += MOE_WAVE * RANK_WAVES) wcnt[i] = 0;
  const long long p0 = (long long)blockIdx.x * RANK_BLOCK_PAIRS + wave * RANK_WAVE_PAIRS + lane;
  int ev[RANK_STEPS], rv[RANK_STEPS];
#pragma unroll
  for (int s = 0; s < RANK_STEPS; ++s) {
    const long long p = p0 + s * MOE_WAVE;
    int e = p < P ? idx[p] : -1;
    ev[s] = p < P ? ((e >= 0 && e < E) ? e : 0) : -1;
  }
  __syncthreads();
  int* cnt = wcnt + wave * E;
  const unsigned long long below_me = (1ull << lane) - 1ull;
#pragma unroll
  for (int s = 0; s < RANK_STEPS; ++s) {
    const bool valid = ev[s] >= 0;
    const int e = valid ? ev[s] : 0;
    // lanes with the same expert id: agree on every bit
    unsigned long long m = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const unsigned long long bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int below = __popcll(m & below_me);
    const int n = __popcll(m);
    // every lane reads the counter before the lowest matching lane writes
    // it (one wavefront's LDS instructions execute in order)
    const int base = valid ? cnt[e] : 0;
    if (valid && below == 0) cnt[e] = base + n;
    rv[s] = base + below;
  }
  __syncthreads();
  // the waves' counts of each expert -> exclusive prefix in wave order
  for (int e = threadIdx.x; e < E; e += MOE_WAVE * RANK_WAVES) {
    int run = 0;
    for (int w = 0; w < RANK_WAVES; ++w) {
      const int v = wcnt[w * E + e];
      wcnt[w * E + e] = run;
      run += v;
    }
    hist[(long long)blockIdx.x * E + e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < RANK_STEPS; ++s)
    if (ev[s] >= 0) local_rank[p0 + s * MOE_WAVE] = cnt[ev[s]] + rv[s];
}

// One workgroup of 1024: hist[b][e] <- sum_{b' < b} hist[b'][e] (the block's
// base inside group e); counts[e] <- sum_b hist[b][e]; offsets = exclusive
// scan of counts (dropless, cap < 0) or e * cap (drop-and-pad), and
// offsets[E] the end.  Thread i scans slice i / E of expert i % E's blocks.
__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* __restrict__ hist, int nblk,
                                                            int E, int cap,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int part[1024];
  __shared__ int buf[1024];
  const int i = threadIdx.x;
  const int S = 1024 / E;   // slices per expert (E <= 1024)
  const int e = i % E, s = i / E;
  const bool on = s < S;
  const int per = (nblk + S - 1) / S;
  const int b0 = on ? s * per : 0, b1 = on ? min(nblk, b0 + per) : 0;
  int sum = 0;
  for (int b = b0; b < b1; ++b) sum += hist[(long long)b * E + e];
  part[i] = sum;
  __syncthreads();
  int run = 0;
  for (int q = 0; q < s && on; ++q) run += part[q * E + e];
  for (int b = b0; b < b1; ++b) {
    const long long o = (long long)b * E + e;
    const int v = hist[o];
    hist[o] = run;
    run += v;
  }
  int tot = 0;
  if (i < E) {
    for (int q = 0; q < S; ++q) tot += part[q * E + i];
    counts[i] = tot;
  }
  buf[i] = tot;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = i >= o ? buf[i - o] : 0;
    __syncthreads();
    buf[i] += add;
    __syncthreads();
  }
  if (i < E) offsets[i] = cap < 0 ? buf[i] - tot : i * cap;
  if (i == E - 1) offsets[E] = cap < 0 ? buf[i] : E * cap;
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

// Row of pair p = (t, j): its stable rank inside expert e is the base of
// p's rank block in group e plus the rank in the block (held in row_id_map
// until now).  Dropless (cap < 0): row = offsets[e] + rank.  Drop-and-pad
// (cap >= 0, offsets[e] = e * cap): the pair keeps that row if rank < cap,
// else it is dropped (-1).
__device__ __forceinline__ long long pair_row(const int32_t* __restrict__ idx,
                                              const int32_t* __restrict__ offsets,
                                              const int32_t* __restrict__ hist,
                                              const int32_t* __restrict__ row_id_map, long long p,
                                              int E, int cap, long long R) {
  int e = idx[p];
  e = (e >= 0 && e < E) ? e : 0;
  const long long b = p / RANK_BLOCK_PAIRS;
  const long long rank = (long long)hist[b * E + e] + row_id_map[p];
  if (cap >= 0 && rank >= cap) return -1;
  long long row = (long long)offsets[e] + rank;
  return row < 0 ? 0 : (row >= R ? R - 1 : row);
}

template <int ESZ>
__global__ __launch_bounds__(ROW_THREADS) void permute_scatter_kernel(
    const void* __restrict__ x, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ hist, int H, int E, int k,
    int cap, long long R, void* __restrict__ xp, int32_t* __restrict__ row_id_map,
    int32_t* __restrict__ src_token) {
  __shared__ uint32_t rofs[MOE_MAX_E];
  const int t = blockIdx.x;
  const uint32_t row_bytes = (uint32_t)H * ESZ;
  for (int j = threadIdx.x; j < k; j += ROW_THREADS) {
    const long long p = (long long)t * k + j;
    const long long row = pair_row(idx, offsets, hist, row_id_map, p, E, cap, R);
    row_id_map[p] = (int)row;
    if (row >= 0) src_token[row] = t;
    rofs[j] = row_off(row, R, row_bytes);
  }
  __syncthreads();
  const int nchunk = row_bytes / 16;
  __amdgpu_buffer_rsrc_t src = make_rsrc((const char*)x + (long long)t * row_bytes, row_bytes);
  __amdgpu_buffer_rsrc_t dst = make_rsrc(xp, rows_bytes(R, row_bytes));
  for (int q0 = 0; q0 < nchunk; q0 += ROW_THREADS * ROW_MAXC) {
    u32x4 v[ROW_MAXC];
#pragma unroll
    for (int i = 0; i < ROW_MAXC; ++i) {
      int q = q0 + i * ROW_THREADS + threadIdx.x;
      v[i] = buf_load16_nt(src, (uint32_t)q * 16u);
    }
    for (int j = 0; j < k; ++j) {
      const uint32_t rb = rofs[j];
#pragma unroll
      for (int i = 0; i < ROW_MAXC; ++i) {
        int q = q0 + i * ROW_THREADS + threadIdx.x;
        if (q < nchunk) buf_store16_nt(dst, rb + (uint32_t)q * 16u, v[i]);
      }
    }
  }
}

// Row map and source tokens only (no row copy): one thread per (t, j).
__global__ __launch_bounds__(256) void permute_maps_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ hist, int T, int E, int k, int cap, long long R,
    int32_t* __restrict__ row_id_map, int32_t* __restrict__ src_token) {
  const long long p = (long long)blockIdx.x * 256 + threadIdx.x;
  if (p >= (long long)T * k) return;
  const int t = (int)(p / k);
  const long long row = pair_row(idx, offsets, hist, row_id_map, p, E, cap, R);
  row_id_map[p] = (int)row;
  if (row >= 0) src_token[row] = t;
}

// Drop-and-pad: the rows [e*C + counts[e], (e+1)*C) that no pair fills get
// src_token = -1 (and zeros in xp when given).  Grid-stride over rows, one
// row per workgroup and pass.
template <int ESZ>
__global__ __launch_bounds__(ROW_THREADS) void permute_pad_kernel(
    const int32_t* __restrict__ counts, int E, int C, int H, void* __restrict__ xp,
    int32_t* __restrict__ src_token) {
  const long long R = (long long)E * C;
  const uint32_t row_bytes = (uint32_t)H * ESZ;
  const int nchunk = row_bytes / 16;
  __amdgpu_buffer_rsrc_t dst = make_rsrc(xp, xp ? rows_bytes(R, row_bytes) : 0u);
  for (long long r = blockIdx.x; r < R; r += gridDim.x) {
    const int e = (int)(r / C), n = (int)(r % C);
    if (n < counts[e]) continue;   // uniform: a filled row
    if (threadIdx.x == 0) src_token[r] = -1;
    if (xp)
      for (int q = threadIdx.x; q < nchunk; q += ROW_THREADS)
        buf_store16(dst, (uint32_t)r * row_bytes + (uint32_t)q * 16u, u32x4{0u, 0u, 0u, 0u});
  }
}

// buf[r, :] = 0 for every row r < R with src_token[r] < 0 (a row no pair
// fills).  Grid-stride over rows, one row per workgroup and pass.
__global__ __launch_bounds__(ROW_THREADS) void clear_empty_rows_kernel(
    const int32_t* __restrict__ src_token, long long R, uint32_t row_bytes, void* __restrict__ buf) {
  const int nchunk = row_bytes / 16;
  __amdgpu_buffer_rsrc_t dst = make_rsrc(buf, rows_bytes(R, row_bytes));
  for (long long r = blockIdx.x; r < R; r += gridDim.x) {
    if (src_token[r] >= 0) continue;   // uniform
    for (int q = threadIdx.x; q < nchunk; q += ROW_THREADS)
      buf_store16(dst, (uint32_t)r * row_bytes + (uint32_t)q * 16u, u32x4{0u, 0u, 0u, 0u});
  }
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
    const T* __restrict__ dxp, const int32_t* __restrict__ row_id_map, int H, int k, long long R,
    const T* __restrict__ add0, const T* __restrict__ add1, T* __restrict__ dx) {
  constexpr int VEC = Elem<T>::VEC;
  __shared__ uint32_t rofs[MOE_MAX_E];
  const int t = blockIdx.x;
  const uint32_t row_bytes = (uint32_t)H * sizeof(T);
  for (int j = threadIdx.x; j < k; j += ROW_THREADS)
    rofs[j] = row_off(row_id_map[(long long)t * k + j], R, row_bytes);
  __syncthreads();
  const int nchunk = row_bytes / 16;
  __amdgpu_buffer_rsrc_t src = make_rsrc(dxp, rows_bytes(R, row_bytes));
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
          const uint32_t rb = rofs[j0 + jj];
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
      if (q < nchunk) buf_store16_nt(out, (uint32_t)q * 16u, pack16(acc[u], T()));
    }
  }
}

// ---------------------------------------------------------------- combine
// y[t] = ys[t] + sum_j gate[t,j] yp[row(t,j)]   (fp32, j ascending)

template <typename T>
__global__ __launch_bounds__(ROW_THREADS) void combine_kernel(
    const T* __restrict__ yp, const int32_t* __restrict__ row_id_map,
    const float* __restrict__ gate, const T* __restrict__ ys, int H, int k, long long R,
    T* __restrict__ y) {
  constexpr int VEC = Elem<T>::VEC;
  __shared__ uint32_t rofs[MOE_MAX_E];
  __shared__ float gates[MOE_MAX_E];
  const int t = blockIdx.x;
  const uint32_t row_bytes = (uint32_t)H * sizeof(T);
  for (int j = threadIdx.x; j < k; j += ROW_THREADS) {
    const long long row = row_id_map[(long long)t * k + j];
    rofs[j] = row_off(row, R, row_bytes);
    // a dropped pair adds nothing (its row reads as zeros; the gate is
    // cleared too so that a non-finite gate cannot leak in)
    gates[j] = (row >= 0 && row < R) ? gate[(long long)t * k + j] : 0.f;
  }
  __syncthreads();
  const int nchunk = row_bytes / 16;
  __amdgpu_buffer_rsrc_t src = make_rsrc(yp, rows_bytes(R, row_bytes));
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
          const uint32_t rb = rofs[j0 + jj];
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
      if (q < nchunk) buf_store16_nt(out, (uint32_t)q * 16u, pack16(acc[u], T()));
    }
  }
}

// dyp[row(t,j)] = gate[t,j] dy[t];  dgate[t,j] = <dy[t], yp[row(t,j)]>
// (per thread fp32 partial dots over its chunks, then a fixed-order
// reduction: wave sums, then the waves in order)
template <typename T>
__global__ __launch_bounds__(ROW_THREADS) void combine_bwd_kernel(
    const T* __restrict__ dy, const T* __restrict__ yp, const int32_t* __restrict__ row_id_map,
    const float* __restrict__ gate, int H, int k, long long R, T* __restrict__ dyp,
    float* __restrict__ dgate) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int NW = ROW_THREADS / MOE_WAVE;
  __shared__ uint32_t rofs[MOE_MAX_E];
  __shared__ float gates[MOE_MAX_E];
  __shared__ float red[ROW_JB][NW];
  const int t = blockIdx.x;
  const uint32_t row_bytes = (uint32_t)H * sizeof(T);
  for (int j = threadIdx.x; j < k; j += ROW_THREADS) {
    // a dropped pair: no dyp row (the stores go past the buffer) and
    // dgate = <dy, 0> = 0
    rofs[j] = row_off(row_id_map[(long long)t * k + j], R, row_bytes);
    gates[j] = gate[(long long)t * k + j];
  }
  __syncthreads();
  const int nchunk = row_bytes / 16;
  __amdgpu_buffer_rsrc_t din = make_rsrc((const char*)dy + (long long)t * row_bytes, row_bytes);
  __amdgpu_buffer_rsrc_t ypr = make_rsrc(yp, rows_bytes(R, row_bytes));
  __amdgpu_buffer_rsrc_t dst = make_rsrc(dyp, rows_bytes(R, row_bytes));
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
          const uint32_t rb = rofs[j0 + jj];
#pragma unroll
          for (int u = 0; u < ROW_QB; ++u)
            v[jj][u] = row_chunk(ypr, rb, threadIdx.x + (c0 + u) * ROW_THREADS, nchunk);
        }
#pragma unroll
      for (int jj = 0; jj < ROW_JB; ++jj)
        if (j0 + jj < k) {
          const uint32_t rb = rofs[j0 + jj];
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
            if (q < nchunk) buf_store16_nt(dst, rb + (uint32_t)q * 16u, pack16(o, T()));
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
  return MOE_OK;
}

// R permuted rows of H elements: addressable below ROW_DROP bytes
static int perm_rows_check(const char* fn, int dt, long long R, int H) {
  if (R < 0) return moe_fail(MOE_ERR_INVALID_ARG, "%s: R = %lld is negative", fn, R);
  MOE_TRY(moe_need_elems(R, H, moe_dt_bytes(dt), fn, "permuted rows"));
  if (R * H * moe_dt_bytes(dt) > (long long)ROW_DROP)
    return moe_fail(MOE_ERR_UNSUPPORTED, "%s: %lld permuted rows of %d elements exceed %u bytes",
                    fn, R, H, ROW_DROP);
  return MOE_OK;
}

extern "C" size_t moe_permute_workspace_bytes(int T, int E, int k) {
  (void)k;
  if (T <= 0 || E <= 0) return 0;
  return (size_t)rank_blocks(T, k) * (size_t)E * sizeof(int32_t);
}

// Dropless (cap < 0, R = T*k) or drop-and-pad (cap = C >= 0, R = E*C).
static int permute_impl(const char* fn, const void* x, int dt, const int32_t* idx, int T, int H,
                        int E, int k, int cap, void* xp, int32_t* counts, int32_t* offsets,
                        int32_t* row_id_map, int32_t* src_token, void* ws, size_t ws_bytes,
                        moe_stream_t stream) {
  MOE_TRY(row_checks(fn, dt, T, H, k));
  MOE_TRY(moe_need_ek(E, k, fn));
  const long long R = cap < 0 ? (long long)T * k : (long long)E * cap;
  MOE_TRY(perm_rows_check(fn, dt, R, H));
  MOE_TRY(moe_need_ptr(counts, fn, "counts", 4));
  MOE_TRY(moe_need_ptr(offsets, fn, "offsets", 4));
  MOE_TRY((xp && T > 0) ? moe_need_ptr(x, fn, "x") : moe_opt_ptr(x, fn, "x"));
  MOE_TRY(moe_opt_ptr(xp, fn, "xp"));
  if (T > 0) {
    MOE_TRY(moe_need_ptr(idx, fn, "idx", 4));
    MOE_TRY(moe_need_ptr(row_id_map, fn, "row_id_map", 4));
    MOE_TRY(moe_need_ptr(ws, fn, "ws", 4));
    if (ws_bytes < moe_permute_workspace_bytes(T, E, k))
      return moe_fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes,
                      moe_permute_workspace_bytes(T, E, k));
  }
  if (R > 0) MOE_TRY(moe_need_ptr(src_token, fn, "src_token", 4));
  hipStream_t s = (hipStream_t)stream;
  int32_t* hist = (int32_t*)ws;
  const int nblk = (int)rank_blocks(T, k);
  if (T > 0) {
    int ebits = 0;
    while ((1 << ebits) < E) ++ebits;
    hipLaunchKernelGGL(permute_rank_kernel, dim3(nblk), dim3(MOE_WAVE * RANK_WAVES),
                       (size_t)RANK_WAVES * E * sizeof(int), s, idx, (long long)T * k, E, ebits,
                       row_id_map, hist);
    MOE_TRY(moe_check_launch(fn));
  }
  // (T = 0: no blocks, so every count is zero -- a fill kernel, not a memset node)
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, hist, nblk, E, cap, counts,
                     offsets);
  MOE_TRY(moe_check_launch(fn));
  if (T > 0) {
    if (xp == nullptr) {
      const long long P = (long long)T * k;
      hipLaunchKernelGGL(permute_maps_kernel, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, s,
                         idx, offsets, hist, T, E, k, cap, R, row_id_map, src_token);
    } else if (dt == MOE_BF16) {
      hipLaunchKernelGGL(permute_scatter_kernel<2>, dim3(T), dim3(ROW_THREADS), 0, s, x, idx,
                         offsets, hist, H, E, k, cap, R, xp, row_id_map, src_token);
    } else {
      hipLaunchKernelGGL(permute_scatter_kernel<4>, dim3(T), dim3(ROW_THREADS), 0, s, x, idx,
                         offsets, hist, H, E, k, cap, R, xp, row_id_map, src_token);
    }
    MOE_TRY(moe_check_launch(fn));
  }
  if (cap > 0) {
    const unsigned grid = (unsigned)(R < 4096 ? R : 4096);
    if (dt == MOE_BF16)
      hipLaunchKernelGGL(permute_pad_kernel<2>, dim3(grid), dim3(ROW_THREADS), 0, s, counts, E,
                         cap, H, xp, src_token);
    else
      hipLaunchKernelGGL(permute_pad_kernel<4>, dim3(grid), dim3(ROW_THREADS), 0, s, counts, E,
                         cap, H, xp, src_token);
    MOE_TRY(moe_check_launch(fn));
  }
  return MOE_OK;
}

extern "C" int moe_permute(const void* x, int dt, const int32_t* idx, int T, int H, int E, int k,
                           void* xp, int32_t* counts, int32_t* offsets, int32_t* row_id_map,
                           int32_t* src_token, void* ws, size_t ws_bytes, moe_stream_t stream) {
  return permute_impl("moe_permute", x, dt, idx, T, H, E, k, -1, xp, counts, offsets, row_id_map,
                      src_token, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- no-allocation permute
// moe_permute with its rank workspace in a file-scope device array instead of
// a caller buffer, for callers that cannot allocate.  The array lives on every
// device the library runs on until the process ends; the rank kernel writes
// every entry a call reads, so nothing has to start at zero.
constexpr long long NOALLOC_SCRATCH_BYTES = 4LL << 20;
static __device__ __align__(256) int32_t scratch[NOALLOC_SCRATCH_BYTES / 4];

// Device address of ``scratch`` on the current device, looked up once per
// device (the array's name is only a host-side stand-in for it).
static int scratch_address(const char* fn, void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return moe_fail(MOE_ERR_LAUNCH, "%s: no current HIP device", fn);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return moe_fail(MOE_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) failed: %s", fn,
                      hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return MOE_OK;
}

extern "C" size_t moe_permute_noalloc_max_scratch_bytes(void) {
  return (size_t)NOALLOC_SCRATCH_BYTES;
}

extern "C" int moe_permute_noalloc(const void* x, int dt, const int32_t* idx, int T, int H, int E,
                                   int k, void* xp, int32_t* counts, int32_t* offsets,
                                   int32_t* row_id_map, int32_t* src_token,
                                   moe_stream_t stream) {
  const char* fn = "moe_permute_noalloc";
  MOE_TRY(row_checks(fn, dt, T, H, k));
  MOE_TRY(moe_need_ek(E, k, fn));
  const size_t need = moe_permute_workspace_bytes(T, E, k);
  if (need > (size_t)NOALLOC_SCRATCH_BYTES)
    return moe_fail(MOE_ERR_UNSUPPORTED,
                    "%s: T = %d, E = %d, k = %d need %zu bytes of rank scratch, above the %lld "
                    "this entry point holds (use moe_permute with a workspace)",
                    fn, T, E, k, need, NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (T > 0) MOE_TRY(scratch_address(fn, &ws));
  return permute_impl(fn, x, dt, idx, T, H, E, k, -1, xp, counts, offsets, row_id_map, src_token,
                      ws, (size_t)NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" int moe_permute_capacity(const void* x, int dt, const int32_t* idx, int T, int H, int E,
                                    int k, int C, void* xp, int32_t* counts, int32_t* offsets,
                                    int32_t* row_id_map, int32_t* src_token, void* ws,
                                    size_t ws_bytes, moe_stream_t stream) {
  const char* fn = "moe_permute_capacity";
  if (C < 0) return moe_fail(MOE_ERR_INVALID_ARG, "%s: C = %d is negative", fn, C);
  return permute_impl(fn, x, dt, idx, T, H, E, k, C, xp, counts, offsets, row_id_map, src_token,
                      ws, ws_bytes, stream);
}

extern "C" int moe_clear_empty_rows(const int32_t* src_token, int R, int dt, int H, void* buf,
                                    moe_stream_t stream) {
  const char* fn = "moe_clear_empty_rows";
  MOE_TRY(moe_need_dt(dt, fn));
  MOE_TRY(moe_need_mult64(H, fn, "H"));
  MOE_TRY(perm_rows_check(fn, dt, R, H));
  if (R == 0) return MOE_OK;
  MOE_TRY(moe_need_ptr(src_token, fn, "src_token", 4));
  MOE_TRY(moe_need_ptr(buf, fn, "buf"));
  const unsigned grid = (unsigned)(R < 4096 ? R : 4096);
  hipLaunchKernelGGL(clear_empty_rows_kernel, dim3(grid), dim3(ROW_THREADS), 0,
                     (hipStream_t)stream, src_token, (long long)R,
                     (uint32_t)(H * moe_dt_bytes(dt)), buf);
  return moe_check_launch(fn);
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
                               int k, int R, const void* add0, const void* add1, void* dx,
                               moe_stream_t stream) {
  const char* fn = "moe_permute_bwd";
  MOE_TRY(row_checks(fn, dt, T, H, k));
  MOE_TRY(perm_rows_check(fn, dt, R, H));
  if (T == 0) return MOE_OK;
  MOE_TRY(moe_need_ptr(dxp, fn, "dxp"));
  MOE_TRY(moe_need_ptr(row_id_map, fn, "row_id_map", 4));
  MOE_TRY(moe_need_ptr(dx, fn, "dx"));
  MOE_TRY(moe_opt_ptr(add0, fn, "add0"));
  MOE_TRY(moe_opt_ptr(add1, fn, "add1"));
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(permute_bwd_kernel<bf16_t>, dim3(T), dim3(ROW_THREADS), 0, s,
                       (const bf16_t*)dxp, row_id_map, H, k, (long long)R, (const bf16_t*)add0,
                       (const bf16_t*)add1, (bf16_t*)dx);
  else
    hipLaunchKernelGGL(permute_bwd_kernel<float>, dim3(T), dim3(ROW_THREADS), 0, s,
                       (const float*)dxp, row_id_map, H, k, (long long)R, (const float*)add0,
                       (const float*)add1, (float*)dx);
  return moe_check_launch(fn);
}

extern "C" int moe_unpermute_combine(const void* yp, const int32_t* row_id_map, const float* gate,
                                     const void* y_shared, int dt, int T, int H, int k, int R,
                                     void* y, moe_stream_t stream) {
  const char* fn = "moe_unpermute_combine";
  MOE_TRY(row_checks(fn, dt, T, H, k));
  MOE_TRY(perm_rows_check(fn, dt, R, H));
  if (T == 0) return MOE_OK;
  MOE_TRY(moe_need_ptr(yp, fn, "yp"));
  MOE_TRY(moe_need_ptr(row_id_map, fn, "row_id_map", 4));
  MOE_TRY(moe_need_ptr(gate, fn, "gate", 4));
  MOE_TRY(moe_opt_ptr(y_shared, fn, "y_shared"));
  MOE_TRY(moe_need_ptr(y, fn, "y"));
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(T), dim3(ROW_THREADS), 0, s,
                       (const bf16_t*)yp, row_id_map, gate, (const bf16_t*)y_shared, H, k,
                       (long long)R, (bf16_t*)y);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(T), dim3(ROW_THREADS), 0, s, (const float*)yp,
                       row_id_map, gate, (const float*)y_shared, H, k, (long long)R,
                       (float*)y);
  return moe_check_launch(fn);
}

extern "C" int moe_unpermute_combine_bwd(const void* dy, const void* yp, const int32_t* row_id_map,
                                         const float* gate, int dt, int T, int H, int k, int R,
                                         void* dyp, float* dgate, moe_stream_t stream) {
  const char* fn = "moe_unpermute_combine_bwd";
  MOE_TRY(row_checks(fn, dt, T, H, k));
  MOE_TRY(perm_rows_check(fn, dt, R, H));
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
                       (const bf16_t*)dy, (const bf16_t*)yp, row_id_map, gate, H, k,
                       (long long)R, (bf16_t*)dyp, dgate);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<float>, dim3(T), dim3(ROW_THREADS), 0, s,
                       (const float*)dy, (const float*)yp, row_id_map, gate, H, k,
                       (long long)R, (float*)dyp, dgate);
  return moe_check_launch(fn);
}
