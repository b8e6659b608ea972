// Grouped SwiGLU GEMMs of the expert layer on gfx950 MFMA
// ([MindSpore-DSv3] 03.3: GroupedMatmul runs every expert's matmul in one
// operator; [Pangu-QA]: the expert backward is split into dX and dW).
//
// One persistent kernel template serves all five products:
//   FWD1  h13 = xp . W13[e]^T, epilogue act = silu(g) * u     (SwiGLU fused)
//   FWD2  yp  = act . W2[e]^T
//   DX1   dact = dyp . W2[e], epilogue SwiGLU backward -> dh13
//   DX2   dxp = dh13 . W13[e]
//   DW    dW[e] = P_e^T . Q_e, contraction over the rows of group e
// A group's rows come from the device offsets table, so the host never
// learns the counts ([MoE-ops] Host-Device section, Fig. 4).
//
// Tiling (the gfx950 counterpart of the staged GM -> L1 -> L0 pipeline and
// the diagonal sub-block assignment of [MoE-ops], MatMul section, Fig. 2):
//  - 256 x 256 output tile per 256-thread workgroup (4 wavefronts as 2 x 2,
//    128 x 128 per wave = 4 x 4 MFMA 32x32 fragments, fp32 accumulators that
//    live in the accumulation registers, one wavefront per SIMD);
//  - K in steps of 128 bytes per row (64 bf16 / 32 fp32), double-buffered in
//    LDS (2 x 64 KB): the next K step is fetched to registers while the MFMAs
//    run on the current one, one barrier per step;
//  - LDS rows of 128 bytes with an XOR swizzle of the 16-byte chunks, so the
//    16-byte fragment reads and the transposed-block writes are spread over
//    the banks without padding;
//  - operands stored MN-major in HBM (weights in dX, both operands in dW) are
//    read as 8x8 (bf16) / 4x4 (fp32) blocks and transposed in registers
//    before the LDS write, so the MFMA always reads K-contiguous fragments;
//  - all global accesses are raw buffer loads/stores whose range is the
//    operand's valid rows: rows past a group's end read as zero and stray
//    writes are dropped by the hardware;
//  - persistent grid of one workgroup per CU; tiles are ordered in bands of
//    8 M-tiles per N-tile, and consecutive tile ids are kept on one XCD
//    (workgroup ids are dealt round-robin over the 8 XCDs), so the
//    workgroups sharing a weight panel share an L2.
#include "validate.hpp"

namespace {

constexpr int BM = 256, BN = 256, NT = 256;
constexpr int WTM = 128, WTN = 128;  // wave tile
constexpr int FM = 4, FN = 4;        // 32x32 fragments per wave tile
constexpr int KCH = BM * 8 / NT;     // K-major 16-byte chunks per thread per operand
constexpr int ROWB = 128;            // bytes per LDS tile row = one K step
constexpr int TILE_BYTES = BM * ROWB;  // 32 KB per operand per stage
constexpr int GM_BAND = 8;           // M-tiles per band in the tile order
constexpr uint32_t OOB = 0x80000000u;  // byte offset past every buffer range

enum Mode { FWD1 = 0, FWD2 = 1, DX1 = 2, DX2 = 3, DW = 4 };

struct GmmArgs {
  const int32_t* offsets;
  int g0, G, R;       // routed groups [g0, g0+G) over R permuted rows
  int shared, shT;    // shared expert group present, and its rows
  int M, N, K, I;     // DW: M x N output, K from rows.  Others: N, K fixed.
  // routed operands
  const void* X; int ldx;                     // row operand (A; DW: P)
  const void* W; int ldw; long long w_gs;     // weights (B) per group; DW: Q rows
  void* C; int ldc; long long c_gs;           // output rows; DW: dW per group
  const void* aux; int ldaux;                 // DX1: h13
  void* C2; int ldc2;                         // FWD1: act
  // shared expert operands (same layouts)
  const void* sX; const void* sW; void* sC; const void* sAux; void* sC2;
};

template <typename T> struct Cfg;
template <> struct Cfg<bf16_t> {
  static constexpr int ES = 2, VEC = 8, BK = 64, KS = 4;  // 4 MFMA k-steps of 16
};
template <> struct Cfg<float> {
  static constexpr int ES = 4, VEC = 4, BK = 32, KS = 16;  // 16 MFMA k-steps of 2
};

__device__ __forceinline__ int lds_off(int row, int chunk) {
  const int swz = (row & 7) ^ ((row >> 3) & 7);
  return row * ROWB + ((chunk ^ swz) << 4);
}

__device__ __forceinline__ f32x16 mfma_step(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_step(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 8x8 bf16 block transpose: in[r] holds 8 values of row r (2 per dword);
// out[c] holds column c's 8 values.
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) w[d] = __builtin_amdgcn_perm(in[2 * d + 1][c >> 1], in[2 * d][c >> 1], sel);
    out[c] = u32x4{w[0], w[1], w[2], w[3]};
  }
}
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[4], u32x4 (&out)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) out[c] = u32x4{in[0][c], in[1][c], in[2][c], in[3][c]};
}

// Operand view: rsrc covers the valid bytes; element (mn, k) lives at
//   K-major:  mn * ld + k        MN-major:  k * ld + mn      (elements)
struct View {
  __amdgpu_buffer_rsrc_t rs;
  int ld;
  int mn_lim;   // mn >= mn_lim reads zero
};

__device__ __forceinline__ View make_view(const void* base, long long bytes, int ld, int mn_lim) {
  View v;
  v.rs = make_rsrc(base, clamp_bytes(bytes));
  v.ld = ld;
  v.mn_lim = mn_lim;
  return v;
}

// ---------------------------------------------------------------- loaders
// K-major tile: 256 rows x 8 chunks, KCH chunks per thread.
template <typename T, bool SWIGLU>
__device__ __forceinline__ void load_kmajor(const View& v, int mn0, int k0, int i0, int I,
                                            u32x4 (&r)[KCH]) {
  constexpr int ES = Cfg<T>::ES, VEC = Cfg<T>::VEC;
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int lin = i * NT + (int)threadIdx.x;
    const int row = lin >> 3, ch = lin & 7;
    int src;
    bool ok;
    if (SWIGLU) {
      // per wave column block of 128 rows: rows [128w, 128w+64) are gate rows
      // i0+64w+c, rows [128w+64, 128w+128) the up rows I+i0+64w+c
      const int w = row >> 7, q = row & 127;
      const int c = w * 64 + (q & 63);
      src = ((q >> 6) ? I : 0) + i0 + c;
      ok = i0 + c < I;
    } else {
      src = mn0 + row;
      ok = src < v.mn_lim;
    }
    const uint32_t off = ok ? (uint32_t)(((long long)src * v.ld + k0 + ch * VEC) * ES) : OOB;
    r[i] = buf_load16(v.rs, off);
  }
}

template <typename T>
__device__ __forceinline__ void store_kmajor(char* lds, const u32x4 (&r)[KCH]) {
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int lin = i * NT + (int)threadIdx.x;
    *(u32x4*)(lds + lds_off(lin >> 3, lin & 7)) = r[i];
  }
}

// MN-major tile: blocks of VEC (k) x VEC (mn); block b: mn-vector b % (256/VEC),
// k-vector b / (256/VEC).
template <typename T>
__device__ __forceinline__ void load_mnmajor(const View& v, int mn0, int k0, int blk,
                                             u32x4 (&r)[Cfg<T>::VEC]) {
  constexpr int ES = Cfg<T>::ES, VEC = Cfg<T>::VEC, NMV = BM / VEC;
  const int mo = blk % NMV, ko = blk / NMV;
  const int mn = mn0 + mo * VEC;
  const bool ok = mn < v.mn_lim;
#pragma unroll
  for (int rr = 0; rr < VEC; ++rr) {
    const int k = k0 + ko * VEC + rr;
    const uint32_t off = ok ? (uint32_t)(((long long)k * v.ld + mn) * ES) : OOB;
    r[rr] = buf_load16(v.rs, off);
  }
}

template <typename T>
__device__ __forceinline__ void store_mnmajor(char* lds, int blk, const u32x4 (&r)[Cfg<T>::VEC]) {
  constexpr int VEC = Cfg<T>::VEC, NMV = BM / VEC;
  const int mo = blk % NMV, ko = blk / NMV;
  u32x4 t[VEC];
  transpose_block(r, t);
#pragma unroll
  for (int c = 0; c < VEC; ++c) *(u32x4*)(lds + lds_off(mo * VEC + c, ko)) = t[c];
}

// ---------------------------------------------------------------- MFMA on one stage
template <typename T>
__device__ __forceinline__ void compute_stage(const char* la, const char* lb, int wm, int wn,
                                              f32x16 (&acc)[FM][FN]) {
  const int lane = threadIdx.x & 63;
  const int r32 = lane & 31, hi = lane >> 5;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int ks = 0; ks < Cfg<T>::KS; ++ks) {
      u32x4 a[FM], b[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f)
        a[f] = *(const u32x4*)(la + lds_off(wm * WTM + f * 32 + r32, ks * 2 + hi));
#pragma unroll
      for (int f = 0; f < FN; ++f)
        b[f] = *(const u32x4*)(lb + lds_off(wn * WTN + f * 32 + r32, ks * 2 + hi));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_step(a[i], b[j], acc[i][j]);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < Cfg<T>::KS; ++ks) {
      const int k = ks * 2 + hi;
      float a[FM], b[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f)
        a[f] = *(const float*)(la + lds_off(wm * WTM + f * 32 + r32, k >> 2) + (k & 3) * 4);
#pragma unroll
      for (int f = 0; f < FN; ++f)
        b[f] = *(const float*)(lb + lds_off(wn * WTN + f * 32 + r32, k >> 2) + (k & 3) * 4);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_step(a[i], b[j], acc[i][j]);
    }
  }
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

// ---------------------------------------------------------------- the kernel
template <typename T, int MODE>
__global__ __launch_bounds__(NT, 1) void gmm_kernel(GmmArgs a) {
  constexpr int ES = Cfg<T>::ES, VEC = Cfg<T>::VEC, BK = Cfg<T>::BK;
  constexpr bool A_MN = (MODE == DW);
  constexpr bool B_MN = (MODE == DX1 || MODE == DX2 || MODE == DW);
  constexpr int NBLK = (BM / VEC) * (ROWB / 16);   // transposed blocks per operand tile

  __shared__ __attribute__((aligned(16))) char smem[4 * TILE_BYTES];
  __shared__ int g_lo[MOE_MAX_E + 2], g_hi[MOE_MAX_E + 2], g_pre[MOE_MAX_E + 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;   // 2 x 2 wave grid
  const int ng = a.G + a.shared;

  // ---- group table: clamped row ranges, then per-group tile prefix (M-var
  // modes) or the group order by descending row count (DW).
  for (int g = tid; g < ng; g += NT) {
    int lo, hi;
    if (g < a.G) {
      lo = a.offsets[a.g0 + g];
      hi = a.offsets[a.g0 + g + 1];
      lo = lo < 0 ? 0 : (lo > a.R ? a.R : lo);
      hi = hi < lo ? lo : (hi > a.R ? a.R : hi);
    } else {
      lo = 0;
      hi = a.shT;
    }
    g_lo[g] = lo;
    g_hi[g] = hi;
  }
  __syncthreads();
  int total;
  int MBt = 0, NBt = 0;
  if constexpr (MODE != DW) {
    if (wave == 0) {
      const int per = (ng + 63) / 64;
      const int b0 = lane * per, b1 = min(ng, b0 + per);
      int s = 0;
      for (int g = b0; g < b1; ++g) s += (g_hi[g] - g_lo[g] + BM - 1) / BM;
      int incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      int run = incl - s;
      for (int g = b0; g < b1; ++g) {
        g_pre[g] = run;
        run += (g_hi[g] - g_lo[g] + BM - 1) / BM;
      }
      if (lane == 63) g_pre[ng] = incl;
    }
    __syncthreads();
    const int nb = (MODE == FWD1) ? (a.I + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
    NBt = nb;
    total = g_pre[ng] * nb;
  } else {
    // stable order by descending row count: g_pre[rank] = g
    for (int g = tid; g < ng; g += NT) {
      const int c = g_hi[g] - g_lo[g];
      int rank = 0;
      for (int h = 0; h < ng; ++h) {
        const int ch = g_hi[h] - g_lo[h];
        rank += (ch > c) || (ch == c && h < g);
      }
      g_pre[rank] = g;
    }
    __syncthreads();
    MBt = (a.M + BM - 1) / BM;
    NBt = (a.N + BN - 1) / BN;
    total = ng * MBt * NBt;
  }

  // ---- persistent loop, XCD-aware workgroup numbering
  const int nwg = gridDim.x;
  const int bid = blockIdx.x;
  const int L = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;

  for (int tile = L; tile < total; tile += nwg) {
    int g, m0, n0, rows0 = 0, rows = 0, kdim;
    if constexpr (MODE != DW) {
      const int MT = g_pre[ng];
      const int band = GM_BAND * NBt;
      const int sup = tile / band, within = tile % band;
      const int first = sup * GM_BAND;
      const int gsz = min(GM_BAND, MT - first);
      const int mi = first + within % gsz;
      const int nbi = within / gsz;
      // group of M-tile mi: last g with g_pre[g] <= mi and a non-empty range
      int lo = 0, hi = ng - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (g_pre[mid] <= mi) lo = mid; else hi = mid - 1;
      }
      g = lo;
      rows0 = g_lo[g] + (mi - g_pre[g]) * BM;
      rows = min(BM, g_hi[g] - rows0);
      m0 = 0;
      n0 = nbi * ((MODE == FWD1) ? BN / 2 : BN);
      kdim = a.K;
    } else {
      const int per = MBt * NBt;
      g = g_pre[tile / per];
      const int local = tile % per;
      const int band = GM_BAND * NBt;
      const int sup = local / band, within = local % band;
      const int first = sup * GM_BAND;
      const int gsz = min(GM_BAND, MBt - first);
      m0 = (first + within % gsz) * BM;
      n0 = (within / gsz) * BN;
      rows0 = g_lo[g];
      kdim = g_hi[g] - g_lo[g];
    }
    g = uniform(g); m0 = uniform(m0); n0 = uniform(n0);
    rows0 = uniform(rows0); rows = uniform(rows); kdim = uniform(kdim);
    const bool sh = g >= a.G;

    // ---- operand views
    View va, vb;
    if constexpr (MODE != DW) {
      const void* xb = sh ? a.sX : a.X;
      va = make_view((const char*)xb + (long long)rows0 * a.ldx * ES, (long long)rows * a.ldx * ES,
                     a.ldx, rows);
      const void* wb = sh ? a.sW : (const void*)((const char*)a.W + (long long)g * a.w_gs * ES);
      const int wrows = (MODE == FWD1) ? 2 * a.I : (B_MN ? a.K : a.N);  // stored rows of W
      const int wcols = B_MN ? a.N : a.K;
      va.mn_lim = rows;
      vb = make_view(wb, (long long)wrows * wcols * ES, a.ldw, B_MN ? a.N : a.N);
    } else {
      const void* pb = sh ? a.sX : a.X;
      const void* qb = sh ? a.sW : a.W;
      va = make_view((const char*)pb + (long long)rows0 * a.ldx * ES, (long long)kdim * a.ldx * ES,
                     a.ldx, a.M);
      vb = make_view((const char*)qb + (long long)rows0 * a.ldw * ES, (long long)kdim * a.ldw * ES,
                     a.ldw, a.N);
    }

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int KT = (kdim + BK - 1) / BK;
    constexpr int BPT = NBLK / NT;   // transposed blocks per thread per operand
    static_assert(BPT * VEC == 8 && KCH == 8, "staging is 8 chunks per operand");
    u32x4 ra[8], rb[8];
    auto fetch = [&](int kt) {
      const int k0 = kt * BK;
      if constexpr (!A_MN) {
        load_kmajor<T, false>(va, m0, k0, 0, 0, ra);
      } else {
#pragma unroll
        for (int b = 0; b < BPT; ++b)
          load_mnmajor<T>(va, m0, k0, b * NT + tid, *(u32x4(*)[VEC]) & ra[b * VEC]);
      }
      if constexpr (!B_MN) {
        load_kmajor<T, MODE == FWD1>(vb, n0, k0, n0, a.I, rb);
      } else {
#pragma unroll
        for (int b = 0; b < BPT; ++b)
          load_mnmajor<T>(vb, n0, k0, b * NT + tid, *(u32x4(*)[VEC]) & rb[b * VEC]);
      }
    };
    auto commit = [&](int stage) {
      char* la = smem + stage * 2 * TILE_BYTES;
      char* lb = la + TILE_BYTES;
      if constexpr (!A_MN) {
        store_kmajor<T>(la, ra);
      } else {
#pragma unroll
        for (int b = 0; b < BPT; ++b)
          store_mnmajor<T>(la, b * NT + tid, *(const u32x4(*)[VEC]) & ra[b * VEC]);
      }
      if constexpr (!B_MN) {
        store_kmajor<T>(lb, rb);
      } else {
#pragma unroll
        for (int b = 0; b < BPT; ++b)
          store_mnmajor<T>(lb, b * NT + tid, *(const u32x4(*)[VEC]) & rb[b * VEC]);
      }
    };

    if (KT > 0) {
      fetch(0);
      commit(0);
      __syncthreads();
    }
    for (int kt = 0; kt < KT; ++kt) {
      const int st = kt & 1;
      if (kt + 1 < KT) fetch(kt + 1);
      compute_stage<T>(smem + st * 2 * TILE_BYTES, smem + st * 2 * TILE_BYTES + TILE_BYTES, wm, wn,
                       acc);
      if (kt + 1 < KT) commit(st ^ 1);
      __syncthreads();
    }

    // ---- epilogue
    const int col = lane & 31;
    const int rsub = (lane >> 5) * 4;
    if constexpr (MODE == FWD1) {
      void* hb = sh ? a.sC : a.C;
      void* ab = sh ? a.sC2 : a.C2;
      const __amdgpu_buffer_rsrc_t hr = make_rsrc((char*)hb + (long long)rows0 * a.ldc * ES,
                                                  clamp_bytes((long long)rows * a.ldc * ES));
      const __amdgpu_buffer_rsrc_t ar = make_rsrc((char*)ab + (long long)rows0 * a.ldc2 * ES,
                                                  clamp_bytes((long long)rows * a.ldc2 * ES));
      // fragments 0,1 of a wave hold gate columns, 2,3 the matching up columns
#pragma unroll
      for (int fn = 0; fn < FN / 2; ++fn) {
        const int i = n0 + wn * (WTN / 2) + fn * 32 + col;
        if (i >= a.I) continue;
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int lr = wm * WTM + f * 32 + (r >> 2) * 8 + rsub + (r & 3);
            if (lr < rows) {
              const float gv = acc[f][fn][r], uv = acc[f][fn + FN / 2][r];
              const float av = gv * sigmoidf_(gv) * uv;
              buf_store_elem<T>(hr, (uint32_t)(lr * a.ldc + i), gv);
              buf_store_elem<T>(hr, (uint32_t)(lr * a.ldc + a.I + i), uv);
              buf_store_elem<T>(ar, (uint32_t)(lr * a.ldc2 + i), av);
            }
          }
      }
    } else if constexpr (MODE == DX1) {
      const void* hb = sh ? a.sAux : a.aux;
      void* db = sh ? a.sC : a.C;
      const __amdgpu_buffer_rsrc_t hr = make_rsrc((const char*)hb + (long long)rows0 * a.ldaux * ES,
                                                  clamp_bytes((long long)rows * a.ldaux * ES));
      const __amdgpu_buffer_rsrc_t dr = make_rsrc((char*)db + (long long)rows0 * a.ldc * ES,
                                                  clamp_bytes((long long)rows * a.ldc * ES));
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int i = n0 + wn * WTN + fn * 32 + col;
        if (i >= a.I) continue;
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int lr = wm * WTM + f * 32 + (r >> 2) * 8 + rsub + (r & 3);
            if (lr < rows) {
              const float gv = buf_load_elem<T>(hr, (uint32_t)(lr * a.ldaux + i));
              const float uv = buf_load_elem<T>(hr, (uint32_t)(lr * a.ldaux + a.I + i));
              const float d = acc[f][fn][r];
              const float s = sigmoidf_(gv);
              buf_store_elem<T>(dr, (uint32_t)(lr * a.ldc + i), d * uv * s * (1.0f + gv * (1.0f - s)));
              buf_store_elem<T>(dr, (uint32_t)(lr * a.ldc + a.I + i), d * gv * s);
            }
          }
      }
    } else {
      // plain store: FWD2 / DX2 rows of C, or DW: dW[g] (M x N)
      void* cb;
      long long cbytes;
      int lim_m;
      if constexpr (MODE == DW) {
        cb = sh ? a.sC : (void*)((char*)a.C + (long long)g * a.c_gs * ES);
        cbytes = (long long)a.M * a.ldc * ES;
        lim_m = a.M;
      } else {
        cb = (char*)(sh ? a.sC : a.C) + (long long)rows0 * a.ldc * ES;
        cbytes = (long long)rows * a.ldc * ES;
        lim_m = rows;
      }
      const __amdgpu_buffer_rsrc_t cr = make_rsrc(cb, clamp_bytes(cbytes));
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int n = n0 + wn * WTN + fn * 32 + col;
        if (n >= a.N) continue;
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int lr = m0 + wm * WTM + f * 32 + (r >> 2) * 8 + rsub + (r & 3);
            if (lr < lim_m) buf_store_elem<T>(cr, (uint32_t)(lr * a.ldc + n), acc[f][fn][r]);
          }
      }
    }
  }
}

// ---------------------------------------------------------------- host side

template <typename T, int MODE>
int launch(const GmmArgs& a, hipStream_t s, const char* what) {
  int grid = moe_cu_count();
  grid = grid >= 8 ? (grid / 8) * 8 : grid;
  hipLaunchKernelGGL((gmm_kernel<T, MODE>), dim3(grid), dim3(NT), 0, s, a);
  return moe_check_launch(what);
}

template <int MODE>
int launch_dt(int dt, const GmmArgs& a, hipStream_t s, const char* what) {
  return dt == MOE_BF16 ? launch<bf16_t, MODE>(a, s, what) : launch<float, MODE>(a, s, what);
}

int gmm_checks(const char* fn, const int32_t* offsets, int g0, int G, int R, int dt, int H, int I,
               const moe_shared_expert* sh) {
  MOE_TRY(moe_need_dt(dt, fn));
  MOE_TRY(moe_need_nonneg(R, fn, "R"));
  MOE_TRY(moe_need_nonneg(g0, fn, "g0"));
  MOE_TRY(moe_need_nonneg(G, fn, "G"));
  if (G > MOE_MAX_E || g0 + G > MOE_MAX_E)
    return moe_fail(MOE_ERR_UNSUPPORTED, "%s: group window [%d, %d) beyond %d experts", fn, g0,
                    g0 + G, MOE_MAX_E);
  MOE_TRY(moe_need_mult64(H, fn, "H"));
  MOE_TRY(moe_need_mult64(I, fn, "I"));
  const int es = moe_dt_bytes(dt);
  MOE_TRY(moe_need_elems(R, H, es, fn, "permuted rows"));
  MOE_TRY(moe_need_elems(R, 2LL * I, es, fn, "h13"));
  MOE_TRY(moe_need_elems(2LL * I, H, es, fn, "one expert's w13"));
  if (G > 0) MOE_TRY(moe_need_ptr(offsets, fn, "offsets", 4));
  if (sh) {
    MOE_TRY(moe_need_nonneg(sh->T, fn, "shared.T"));
    MOE_TRY(moe_need_elems(sh->T, H, es, fn, "shared rows"));
    MOE_TRY(moe_need_elems(sh->T, 2LL * I, es, fn, "shared h13"));
  }
  return MOE_OK;
}

GmmArgs base_args(const int32_t* offsets, int g0, int G, int R, const moe_shared_expert* sh) {
  GmmArgs a = {};
  a.offsets = offsets;
  a.g0 = g0;
  a.G = G;
  a.R = R;
  a.shared = (sh && sh->T > 0) ? 1 : 0;
  a.shT = a.shared ? sh->T : 0;
  return a;
}

}  // namespace

extern "C" int moe_grouped_gemm_fwd(const void* xp, const int32_t* offsets, int g0, int G, int R,
                                    int dt, int H, int I, const void* w13, const void* w2,
                                    void* h13, void* act, void* yp,
                                    const moe_shared_expert* sh, moe_stream_t stream) {
  const char* fn = "moe_grouped_gemm_fwd";
  MOE_TRY(gmm_checks(fn, offsets, g0, G, R, dt, H, I, sh));
  if (G > 0 && R > 0) {
    MOE_TRY(moe_need_ptr(xp, fn, "xp"));
    MOE_TRY(moe_need_ptr(w13, fn, "w13"));
    MOE_TRY(moe_need_ptr(w2, fn, "w2"));
    MOE_TRY(moe_need_ptr(h13, fn, "h13"));
    MOE_TRY(moe_need_ptr(act, fn, "act"));
    MOE_TRY(moe_need_ptr(yp, fn, "yp"));
  }
  const bool use_sh = sh && sh->T > 0;
  if (use_sh) {
    MOE_TRY(moe_need_ptr(sh->x, fn, "shared.x"));
    MOE_TRY(moe_need_ptr(sh->w13, fn, "shared.w13"));
    MOE_TRY(moe_need_ptr(sh->w2, fn, "shared.w2"));
    MOE_TRY(moe_need_ptr(sh->h13, fn, "shared.h13"));
    MOE_TRY(moe_need_ptr(sh->act, fn, "shared.act"));
    MOE_TRY(moe_need_ptr(sh->y, fn, "shared.y"));
  }
  if (!use_sh && (G == 0 || R == 0)) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  GmmArgs a = base_args(offsets, g0, (R > 0) ? G : 0, R, sh);
  // FWD1: h13 = X . W13^T (N = 2I as I gate/up pairs, K = H)
  a.N = 2 * I; a.K = H; a.I = I;
  a.X = xp; a.ldx = H;
  a.W = w13; a.ldw = H; a.w_gs = 2LL * I * H;
  a.C = h13; a.ldc = 2 * I;
  a.C2 = act; a.ldc2 = I;
  if (use_sh) { a.sX = sh->x; a.sW = sh->w13; a.sC = sh->h13; a.sC2 = sh->act; }
  MOE_TRY(launch_dt<FWD1>(dt, a, s, fn));
  // FWD2: yp = act . W2^T (N = H, K = I)
  a.N = H; a.K = I;
  a.X = act; a.ldx = I;
  a.W = w2; a.ldw = I; a.w_gs = (long long)H * I;
  a.C = yp; a.ldc = H;
  a.C2 = nullptr;
  if (use_sh) { a.sX = sh->act; a.sW = sh->w2; a.sC = sh->y; a.sC2 = nullptr; }
  return launch_dt<FWD2>(dt, a, s, fn);
}

extern "C" int moe_grouped_gemm_bwd_dx(const void* dyp, const int32_t* offsets, int g0, int G,
                                       int R, int dt, int H, int I, const void* w13,
                                       const void* w2, const void* h13, void* dh13, void* dxp,
                                       const moe_shared_expert* sh, moe_stream_t stream) {
  const char* fn = "moe_grouped_gemm_bwd_dx";
  MOE_TRY(gmm_checks(fn, offsets, g0, G, R, dt, H, I, sh));
  if (G > 0 && R > 0) {
    MOE_TRY(moe_need_ptr(dyp, fn, "dyp"));
    MOE_TRY(moe_need_ptr(w13, fn, "w13"));
    MOE_TRY(moe_need_ptr(w2, fn, "w2"));
    MOE_TRY(moe_need_ptr(h13, fn, "h13"));
    MOE_TRY(moe_need_ptr(dh13, fn, "dh13"));
    MOE_TRY(moe_need_ptr(dxp, fn, "dxp"));
  }
  const bool use_sh = sh && sh->T > 0;
  if (use_sh) {
    MOE_TRY(moe_need_ptr(sh->dy, fn, "shared.dy"));
    MOE_TRY(moe_need_ptr(sh->w13, fn, "shared.w13"));
    MOE_TRY(moe_need_ptr(sh->w2, fn, "shared.w2"));
    MOE_TRY(moe_need_ptr(sh->h13, fn, "shared.h13"));
    MOE_TRY(moe_need_ptr(sh->dh13, fn, "shared.dh13"));
    MOE_TRY(moe_need_ptr(sh->dx, fn, "shared.dx"));
  }
  if (!use_sh && (G == 0 || R == 0)) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  GmmArgs a = base_args(offsets, g0, (R > 0) ? G : 0, R, sh);
  // DX1: dact = dyp . W2 (W2 stored [K=H][N=I]), SwiGLU backward into dh13
  a.N = I; a.K = H; a.I = I;
  a.X = dyp; a.ldx = H;
  a.W = w2; a.ldw = I; a.w_gs = (long long)H * I;
  a.C = dh13; a.ldc = 2 * I;
  a.aux = h13; a.ldaux = 2 * I;
  if (use_sh) { a.sX = sh->dy; a.sW = sh->w2; a.sC = sh->dh13; a.sAux = sh->h13; }
  MOE_TRY(launch_dt<DX1>(dt, a, s, fn));
  // DX2: dxp = dh13 . W13 (W13 stored [K=2I][N=H])
  a.N = H; a.K = 2 * I;
  a.X = dh13; a.ldx = 2 * I;
  a.W = w13; a.ldw = H; a.w_gs = 2LL * I * H;
  a.C = dxp; a.ldc = H;
  a.aux = nullptr;
  if (use_sh) { a.sX = sh->dh13; a.sW = sh->w13; a.sC = sh->dx; a.sAux = nullptr; }
  return launch_dt<DX2>(dt, a, s, fn);
}

extern "C" int moe_grouped_gemm_bwd_dw(const void* xp, const void* act, const void* dyp,
                                       const void* dh13, const int32_t* offsets, int g0, int G,
                                       int R, int dt, int H, int I, void* dw13, void* dw2,
                                       const moe_shared_expert* sh, moe_stream_t stream) {
  const char* fn = "moe_grouped_gemm_bwd_dw";
  MOE_TRY(gmm_checks(fn, offsets, g0, G, R, dt, H, I, sh));
  if (G > 0) {
    MOE_TRY(moe_need_ptr(dw13, fn, "dw13"));
    MOE_TRY(moe_need_ptr(dw2, fn, "dw2"));
    if (R > 0) {
      MOE_TRY(moe_need_ptr(xp, fn, "xp"));
      MOE_TRY(moe_need_ptr(act, fn, "act"));
      MOE_TRY(moe_need_ptr(dyp, fn, "dyp"));
      MOE_TRY(moe_need_ptr(dh13, fn, "dh13"));
    }
  }
  const bool use_sh = sh && sh->T >= 0 && (sh->dw13 || sh->dw2);
  if (use_sh) {
    MOE_TRY(moe_need_ptr(sh->dw13, fn, "shared.dw13"));
    MOE_TRY(moe_need_ptr(sh->dw2, fn, "shared.dw2"));
    if (sh->T > 0) {
      MOE_TRY(moe_need_ptr(sh->x, fn, "shared.x"));
      MOE_TRY(moe_need_ptr(sh->act, fn, "shared.act"));
      MOE_TRY(moe_need_ptr(sh->dy, fn, "shared.dy"));
      MOE_TRY(moe_need_ptr(sh->dh13, fn, "shared.dh13"));
    }
  }
  if (!use_sh && G == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  GmmArgs a = base_args(offsets, g0, G, R, sh);
  a.shared = use_sh ? 1 : 0;   // an empty shared expert still gets zero gradients
  a.shT = use_sh ? sh->T : 0;
  // dW2[e] [H,I] = dyp_e^T . act_e
  a.M = H; a.N = I; a.I = I;
  a.X = dyp; a.ldx = H;
  a.W = act; a.ldw = I;
  a.C = dw2; a.ldc = I; a.c_gs = (long long)H * I;
  if (use_sh) { a.sX = sh->dy; a.sW = sh->act; a.sC = sh->dw2; }
  MOE_TRY(launch_dt<DW>(dt, a, s, fn));
  // dW13[e] [2I,H] = dh13_e^T . xp_e
  a.M = 2 * I; a.N = H;
  a.X = dh13; a.ldx = 2 * I;
  a.W = xp; a.ldw = H;
  a.C = dw13; a.ldc = H; a.c_gs = 2LL * I * H;
  if (use_sh) { a.sX = sh->dh13; a.sW = sh->x; a.sC = sh->dw13; }
  return launch_dt<DW>(dt, a, s, fn);
}
