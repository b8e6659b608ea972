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
// the diagonal sub-block assignment of [MoE-ops], MatMul section, Fig. 2, and
// of the load / compute / store pipeline of [CANN-MoE] s2.2):
//  - 256 x 256 output tile per 256-thread workgroup (4 wavefronts as 2 x 2,
//    128 x 128 per wave = 4 x 4 MFMA 32x32 fragments, fp32 accumulators in
//    the accumulation registers, one wavefront per SIMD);
//  - K in steps of 64 bytes per row (32 bf16 / 16 fp32) through a ring of 4
//    LDS stages (4 x 32 KB).  Tiles are copied HBM -> LDS by the buffer
//    load-to-LDS path (no staging registers, no LDS store instructions) three
//    steps ahead of the MFMAs, so three K steps of loads are in flight while
//    one is multiplied;
//  - an operand stored K-contiguous (activations, forward weights) sits in
//    LDS as 256 rows of 64 bytes with the 16-byte chunks XOR-swizzled by row;
//    an operand stored MN-contiguous (weights in dX, both operands in dW)
//    sits as K rows of 256 elements, and the MFMA fragments are read with the
//    gfx950 LDS transpose read (ds_read_b64_tr_b16), so no operand is ever
//    transposed in registers or in HBM;
//  - all global accesses are raw buffer accesses whose range is the operand's
//    valid rows: rows past a group's end read as zero and stray writes are
//    dropped by the hardware;
//  - persistent grid of one workgroup per CU; tiles are ordered in bands of
//    8 M-tiles per N-tile, and consecutive tile ids are kept on one XCD
//    (workgroup ids are dealt round-robin over the 8 XCDs), so the
//    workgroups sharing a weight panel share an L2.
#include <type_traits>

#include "validate.hpp"

namespace {

constexpr int BM = 256, BN = 256;
constexpr int WTM = 128;             // wave tile rows (two wave rows per tile)
constexpr int FM = 4;                // 32-row fragments per wave tile

// W wavefronts per workgroup in WM wave rows x W/WM wave columns over a
// tile of WM * 128 rows and 256 columns.  W = 4, WM = 2 gives each wave a
// 128 x 128 tile (4 x 4 fragments, accumulators in the AGPRs, one wave per
// SIMD); W = 8 gives 128 x 64 (4 x 2 fragments, two waves per SIMD, so one
// wave's MFMAs run while the other waits on LDS or a barrier).  W = 4,
// WM = 1 is the strip tile for row tiles of at most 128 rows: one row of
// four 128 x 64 waves, so a short row tile costs half a tile, not a whole
// one with two waves on padding.
template <int W, int WM = 2>
struct Waves {
  static constexpr int NT = 64 * W;       // threads per workgroup
  static constexpr int WN = W / WM;       // wave columns
  static constexpr int FN = 8 / WN;       // 32-column fragments per wave tile
  static constexpr int WTN = 32 * FN;     // wave tile columns
  static constexpr int HW = WTN / 2;      // a wave's columns in one epilogue slice
  static constexpr int BMT = WM * 128;    // tile rows
};
constexpr int RING_BYTES = 131072;   // LDS ring of operand stages (also the epilogue slice)
constexpr int GM_BAND = 8;           // M-tiles per band in the tile order
constexpr int EP_PITCH = 128;        // floats per LDS row of an epilogue slice (128 KB in all)
constexpr uint32_t OOB = 0x80000000u;  // byte offset past every operand range (loads)
// Byte offset of a dropped store: past every output range, whose descriptor
// sizes are capped by out_bytes(); the epilogues compute a store's offset
// with this in place of a branch, so they stay free of divergent control flow.
constexpr uint32_t DROP = 0xFFFFFFF0u;
__host__ __device__ __forceinline__ uint32_t out_bytes(long long b) {
  return b <= 0 ? 0u : (b >= 0xFFFFFFE0LL ? 0xFFFFFFE0u : (uint32_t)b);
}

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
  // dense groups: all G groups have rows [0, shT) and their own operands at
  // X + g*x_gs, W + g*w_gs, C + g*c_gs (elements); no offsets table
  int dense; long long x_gs;
  int krep;      // > 1: each A K step serves krep consecutive K steps, whose
                 // B rows differ (the parts of a split fp32 operand)
  int out_f32;   // plain-store epilogue writes fp32 whatever T is
  // tile scheduler counters (NULL: static tile order): 8 per-XCD tile
  // counters and a finished-workgroup counter, zero on entry and on exit
  int* cnt;
  // row gather (kernels built with GATHER): routed row r of the token
  // operand is row gather[r] of X (gather_rows rows) instead of row r --
  // FWD1's A rows, DW's Q rows (the K rows of the second factor)
  const int32_t* gather; int gather_rows;
};

// Per element type: K step BK (KS MFMA k-steps), ring of STAGES stages of two
// OPB-byte operand tiles, ROWB bytes per K-major tile row.
template <typename T> struct Cfg;
template <> struct Cfg<bf16_t> {
  static constexpr int ES = 2, VEC = 8, BK = 32, KS = 2;   // 2 MFMA k-steps of 16
  static constexpr int STAGES = 4, OPB = 16384, ROWB = 64;
};
template <> struct Cfg<float> {
  static constexpr int ES = 4, VEC = 4, BK = 16, KS = 8;   // 8 MFMA k-steps of 2
  static constexpr int STAGES = 4, OPB = 16384, ROWB = 64;
};
// 1 KB copies per wave per operand per K step
template <typename T, int W> constexpr int DPO_OF = Cfg<T>::OPB / 1024 / W;

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_t;

// K-major stage tile: 256 rows x ROWB bytes; 16-byte chunk c of row r lives
// in slot c ^ kswz(r), so the 16 rows that one pass of a 16-byte LDS read
// serves (16 lanes, 256 bytes of banks) hit 16 distinct bank groups.
template <typename T> __device__ __forceinline__ int kswz(int row) {
  static_assert(Cfg<T>::ROWB == 64, "64-byte rows: 4 rows per 256 bytes of banks");
  return (row >> 2) & 3;
}
template <typename T> __device__ __forceinline__ int kslot_off(int row, int chunk) {
  return row * Cfg<T>::ROWB + ((chunk ^ kswz<T>(row)) << 4);
}
// MN-major stage tile (bf16): 32 K rows x 512 bytes; 16-byte chunk c of row k
// lives in slot c ^ (4 * (k & 3)), so the four rows of one transpose read
// land in distinct bank groups.
__device__ __forceinline__ int mslot_off_bf16(int k, int chunk) {
  return k * 512 + ((chunk ^ ((k & 3) << 2)) << 4);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char_t;

// Raw buffer descriptor as four SGPR words (range-checked, stride 0).
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, uint32_t bytes) {
  const unsigned long long b = (unsigned long long)base;
  return i32x4{uniform((int)(uint32_t)b), uniform((int)((b >> 32) & 0xffffu)), uniform((int)bytes),
               MOE_RSRC_DW3};
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const lds_char_t*)p;
}

// One 1 KB HBM -> LDS copy: lane l's 16 bytes at voff + soff land at
// lds + 16 l.  Issued as inline assembly so that the compiler does not guard
// every later LDS read with a wait on all outstanding copies; the kernel
// waits for exactly the copies it needs (wait_vm) before a barrier.  The LDS
// address goes through M0, and an LDS-DMA load needs one wait state after
// the write of M0 (the compiler's hazard checks do not look inside inline
// assembly): M0 is written here, followed by s_nop 0.  Without the nop, a
// copy issued right after its M0 write could land at the previous copy's
// LDS address (seen as wrong, non-deterministic weight gradients whenever
// the scheduler put the two instructions back to back).
__device__ __forceinline__ void dma16(const i32x4& rs, uint32_t lds, uint32_t voff, int soff) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(uniform(soff)), "s"(uniform((int)lds))
               : "memory", "m0");
}

// Wait until at most n of this wave's buffer loads are outstanding.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ f32x16 mfma_step(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_step(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Operand view: rsrc covers the valid bytes; element (mn, k) lives at
//   K-major:  mn * ld + k        MN-major:  k * ld + mn      (elements)
struct View {
  i32x4 rs;
  int ld;
  int mn_lim;   // mn >= mn_lim reads zero
};

__device__ __forceinline__ View make_view(const void* base, long long bytes, int ld, int mn_lim) {
  View v;
  v.rs = raw_rsrc(base, clamp_bytes(bytes));
  v.ld = ld;
  v.mn_lim = mn_lim;
  return v;
}

// ---------------------------------------------------------------- HBM -> LDS
// One operand tile of one K step is OPB / 1 KB copies, DPO per wave.  The
// per-lane byte offsets of a tile are fixed; a K step only moves the uniform
// offset (k0 * ES for K-major, k0 * ld * ES for MN-major).
//
// K-major: a copy covers 1024 / ROWB whole rows; lane l fills row
// q * RPC + l / LPR, slot l % LPR, from the chunk that belongs in that slot.
template <typename T, bool SWIGLU, int WTN, int DPO>
__device__ __forceinline__ void kmajor_offsets(const View& v, int mn0, int I,
                                               uint32_t (&off)[DPO]) {
  constexpr int ES = Cfg<T>::ES, VEC = Cfg<T>::VEC, HW = WTN / 2;
  constexpr int LPR = Cfg<T>::ROWB / 16, RPC = 64 / LPR;   // lanes per row, rows per copy
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < DPO; ++j) {
    const int q = wave * DPO + j;
    const int row = q * RPC + lane / LPR;
    const int chunk = (lane % LPR) ^ kswz<T>(row);
    int src;
    bool ok;
    if (SWIGLU) {
      // per wave column block of WTN rows: rows [WTN w, WTN w + HW) are gate
      // rows i0 + HW w + c, the next HW rows the up rows I + i0 + HW w + c
      // (i0 = mn0)
      const int w = row / WTN, r = row % WTN;
      const int c = w * HW + (r % HW);
      src = ((r / HW) ? I : 0) + mn0 + c;
      ok = mn0 + c < I;
    } else {
      src = mn0 + row;
      ok = src < v.mn_lim;
    }
    off[j] = ok ? (uint32_t)(((long long)src * v.ld + chunk * VEC) * ES) : OOB;
  }
}

// MN-major: bf16 copy q covers K rows 2q, 2q+1 (lane l: row 2q + l/32, slot
// l%32); fp32 copy q covers K row q (lane l: slot l).
template <typename T, int DPO>
__device__ __forceinline__ void mnmajor_offsets(const View& v, int mn0, uint32_t (&off)[DPO]) {
  constexpr int ES = Cfg<T>::ES, VEC = Cfg<T>::VEC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < DPO; ++j) {
    const int q = wave * DPO + j;
    int k, chunk;
    if constexpr (sizeof(T) == 2) {
      k = 2 * q + (lane >> 5);
      chunk = (lane & 31) ^ ((k & 3) << 2);
    } else {
      k = q;
      chunk = lane;
    }
    const int mn = mn0 + chunk * VEC;
    off[j] = mn < v.mn_lim ? (uint32_t)(((long long)k * v.ld + mn) * ES) : OOB;
  }
}

// K-major, rows gathered: tile row `row` (< rows) is row gather[rows0 + row]
// of the view; the indices are read once per tile.
template <typename T, int DPO>
__device__ __forceinline__ void kmajor_offsets_gather(const View& v, const int32_t* gather,
                                                      int rows0, int rows, uint32_t (&off)[DPO]) {
  constexpr int ES = Cfg<T>::ES, VEC = Cfg<T>::VEC;
  constexpr int LPR = Cfg<T>::ROWB / 16, RPC = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t gi = make_rsrc(gather + rows0, (uint32_t)rows * 4u);
  int src[DPO];
#pragma unroll
  for (int j = 0; j < DPO; ++j) {
    const int row = (wave * DPO + j) * RPC + lane / LPR;
    src[j] = (int)buf_load4(gi, (uint32_t)row * 4u);    // row >= rows reads 0, masked below
  }
#pragma unroll
  for (int j = 0; j < DPO; ++j) {
    const int row = (wave * DPO + j) * RPC + lane / LPR;
    const int chunk = (lane % LPR) ^ kswz<T>(row);
    off[j] = row < rows ? (uint32_t)src[j] * (uint32_t)(v.ld * ES) + (uint32_t)(chunk * VEC * ES)
                        : OOB;
  }
}

// One 256-byte HBM -> LDS copy of 4-byte words: lane l's word at voff + soff
// lands at lds + 4 l (the row indices of a gathered operand).
__device__ __forceinline__ void dma4(const i32x4& rs, uint32_t lds, uint32_t voff, int soff) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(uniform(soff)), "s"(uniform((int)lds))
               : "memory", "m0");
}

template <int DPO>
__device__ __forceinline__ void issue_op(const View& v, const char* lds_op,
                                         const uint32_t (&off)[DPO], int soff) {
  const int wave = threadIdx.x >> 6;
  const uint32_t base = lds_addr(lds_op) + wave * DPO * 1024;
#pragma unroll
  for (int j = 0; j < DPO; ++j) dma16(v.rs, base + j * 1024, off[j], soff);
}

// ---------------------------------------------------------------- LDS -> MFMA
// Fragment f of a wave: 32 rows (M or N) starting at r0, K step ks.
// bf16 lane l holds elements k = 16 ks + 8 (l/32) + 0..7 of row r0 + l%32.
template <typename T, bool MN>
__device__ __forceinline__ auto read_frag(const char* lds, int r0, int ks) {
  const int lane = threadIdx.x & 63;
  if constexpr (sizeof(T) == 2) {
    if constexpr (!MN) {
      return *(const u32x4*)(lds + kslot_off<T>(r0 + (lane & 31), ks * 2 + (lane >> 5)));
    } else {
      // transpose read: in a group of 16 lanes, lane i points at row k0 + i/4,
      // columns c0 + 4 (i%4) .. +3 and receives column c0 + i of rows k0..k0+3
      const int g = lane >> 4, i = lane & 15;
      const int c0 = r0 + (g & 1) * 16;
      const int kb = ks * 16 + (g >> 1) * 8 + (i >> 2);
      const int col = c0 + 4 * (i & 3);
      const char* p0 = lds + mslot_off_bf16(kb, col >> 3) + (col & 7) * 2;
      const char* p1 = lds + mslot_off_bf16(kb + 4, col >> 3) + (col & 7) * 2;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t)(p0));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t)(p1));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{l2.x, l2.y, h2.x, h2.y};
    }
  } else {
    const int k = ks * 2 + (lane >> 5);
    const int r = r0 + (lane & 31);
    if constexpr (!MN) {
      return *(const float*)(lds + kslot_off<T>(r, k >> 2) + (k & 3) * 4);
    } else {
      return *(const float*)(lds + k * 1024 + r * 4);
    }
  }
}

// The MFMA takes the B fragment as its first operand, so accumulator register
// r of fragment (i, j) holds C[m][n] with m = 32 i + lane%32 and
// n = 32 j + 8 (r/4) + 4 (lane/32) + r%4: every lane owns runs of four
// consecutive output columns, which the epilogue writes to LDS as one
// 16-byte store.
template <typename T, bool A_MN, bool B_MN, int W, int WM>
struct Frags {
  static constexpr int FN = Waves<W, WM>::FN, WTN = Waves<W, WM>::WTN;
  decltype(read_frag<T, A_MN>(nullptr, 0, 0)) a[FM];
  decltype(read_frag<T, B_MN>(nullptr, 0, 0)) b[FN];
  __device__ __forceinline__ void load(const char* la, const char* lb, int wm, int wn, int ks) {
#pragma unroll
    for (int f = 0; f < FM; ++f) a[f] = read_frag<T, A_MN>(la, wm * WTM + f * 32, ks);
#pragma unroll
    for (int f = 0; f < FN; ++f) b[f] = read_frag<T, B_MN>(lb, wn * WTN + f * 32, ks);
  }
  // fragment q of a load: q < FM is A fragment q, else B fragment q - FM
  __device__ __forceinline__ void load1(const char* la, const char* lb, int wm, int wn, int ks,
                                        int q) {
    if (q < FM) a[q] = read_frag<T, A_MN>(la, wm * WTM + q * 32, ks);
    else b[q - FM] = read_frag<T, B_MN>(lb, wn * WTN + (q - FM) * 32, ks);
  }
  __device__ __forceinline__ void mma(f32x16 (&acc)[FM][FN]) const {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma_step(b[j], a[i], acc[i][j]);
  }
};

// logistic function: hardware exp2 and reciprocal (about 2 ulp), no IEEE divide
__device__ __forceinline__ float sigmoidf_(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// act = silu(g) * u from the gate and up values as h13 stores them (rounded
// to T), so the backward's derivative and a recomputed act see the very
// same g and u as the forward
template <typename T>
__device__ __forceinline__ float swiglu_act(float g, float u) {
  if constexpr (sizeof(T) == 2) {
    g = bf16_to_f32(f32_to_bf16(g));
    u = bf16_to_f32(f32_to_bf16(u));
  }
  return g * sigmoidf_(g) * u;
}

// ---------------------------------------------------------------- tile spaces
// Group window of a launch in LDS (the products of one launch share it).
struct GroupLds {
  int lo[MOE_MAX_E + 2], hi[MOE_MAX_E + 2];   // clamped row ranges
  int pre[MOE_MAX_E + 2];   // row-tiled products: M-tiles before each group, pre[ng] = all
  int ord[MOE_MAX_E + 2];   // weight-gradient products: groups by descending row count
};

// Tile space of one product.
struct Space {
  int total;       // tiles
  int MBt, NBt;    // DW: M and N tiles of a group; others: N tiles of a row tile
  bool light;      // LIGHT builds: the per-fragment-count loops are in use
};

// Row ranges of the window's groups (and of the shared expert as group G).
__device__ __forceinline__ void load_groups(const GmmArgs& a, GroupLds& gl) {
  const int ng = a.G + a.shared;
  for (int g = threadIdx.x; g < ng; g += blockDim.x) {
    int lo, hi;
    if (g < a.G && !a.dense) {
      lo = a.offsets[a.g0 + g];
      hi = a.offsets[a.g0 + g + 1];
      lo = lo < 0 ? 0 : (lo > a.R ? a.R : lo);
      hi = hi < lo ? lo : (hi > a.R ? a.R : hi);
    } else {
      lo = 0;
      hi = a.shT;
    }
    gl.lo[g] = lo;
    gl.hi[g] = hi;
  }
  __syncthreads();
}

// Per-group M-tile prefix (row-tiled modes) into gl.pre.
__device__ __forceinline__ void tile_prefix(int ng, GroupLds& gl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    const int per = (ng + 63) / 64;
    const int b0 = lane * per, b1 = min(ng, b0 + per);
    int s = 0;
    for (int g = b0; g < b1; ++g) s += (gl.hi[g] - gl.lo[g] + BM - 1) / BM;
    int incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int run = incl - s;
    for (int g = b0; g < b1; ++g) {
      gl.pre[g] = run;
      run += (gl.hi[g] - gl.lo[g] + BM - 1) / BM;
    }
    if (lane == 63) gl.pre[ng] = incl;
  }
  __syncthreads();
}

// Group order by descending row count (stable) into gl.ord.
__device__ __forceinline__ void group_order(int ng, GroupLds& gl) {
  for (int g = threadIdx.x; g < ng; g += blockDim.x) {
    const int c = gl.hi[g] - gl.lo[g];
    int rank = 0;
    for (int h = 0; h < ng; ++h) {
      const int ch = gl.hi[h] - gl.lo[h];
      rank += (ch > c) || (ch == c && h < g);
    }
    gl.ord[rank] = g;
  }
  __syncthreads();
}

// Tile space of a product whose group tables are in place (tile_prefix for
// row-tiled modes, group_order for DW).  s_tmp: an LDS int free until the
// first epilogue.
template <int MODE, bool LIGHT>
__device__ __forceinline__ Space tile_space(const GmmArgs& a, const GroupLds& gl, int* s_tmp) {
  const int ng = a.G + a.shared;
  Space sp;
  sp.light = false;
  if constexpr (MODE != DW) {
    sp.MBt = 0;
    sp.NBt = (MODE == FWD1) ? (a.I + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
    sp.total = gl.pre[ng] * sp.NBt;
    if constexpr (LIGHT) {
      // light builds in use where at least half of the M-tiles are light (a
      // group's last M-tile holding at most 64 rows): a few light tiles among
      // full ones finish early, let some XCDs run ahead of the others and
      // widen the stretch of operand panels the chip works on (HBM reads of
      // the Pangu share's launches grew by 7-63% for no gain in time)
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      if (wave == 0) {
        int lt = 0;
        for (int g = lane; g < ng; g += 64) {
          const int r = gl.hi[g] - gl.lo[g];
          lt += (r > 0 && r - (r - 1) / BM * BM <= 64);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) lt += __shfl_xor(lt, o, 64);
        if (lane == 0) *s_tmp = lt;
      }
      __syncthreads();
      sp.light = 2 * *s_tmp >= gl.pre[ng];
      __syncthreads();
    }
  } else {
    sp.MBt = (a.M + BM - 1) / BM;
    sp.NBt = (a.N + BN - 1) / BN;
    sp.total = ng * sp.MBt * sp.NBt;
  }
  return sp;
}

// ---------------------------------------------------------------- one tile
// Row tile tile_id of a row-tiled product: group g, rows [rows0, rows0 +
// rows) (rows <= BM) and N-tile nbi, in band order: GM_BAND M-tiles at a
// time, every N-tile of them, M fastest.
struct RowTile {
  int g, rows0, rows, nbi;
};
__device__ __forceinline__ RowTile locate_row_tile(const GroupLds& gl, const Space& sp, int ng,
                                                   int tile) {
  const int MT = gl.pre[ng];
  const int band = GM_BAND * sp.NBt;
  const int sup = tile / band, within = tile % band;
  const int first = sup * GM_BAND;
  const int gsz = min(GM_BAND, MT - first);
  const int mi = first + within % gsz;
  RowTile rt;
  rt.nbi = within / gsz;
  // group of M-tile mi: last g with pre[g] <= mi and a non-empty range
  int lo = 0, hi = ng - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (gl.pre[mid] <= mi) lo = mid; else hi = mid - 1;
  }
  rt.g = lo;
  rt.rows0 = gl.lo[lo] + (mi - gl.pre[lo]) * BM;
  rt.rows = min(BM, gl.hi[lo] - rt.rows0);
  return rt;
}

// Weight-gradient tile tile_id: its group (in descending row order), the
// corner of its M x N block and the group's rows (the K range).
struct DwLoc {
  int g, m0, n0, rows0, kdim;
};
__device__ __forceinline__ DwLoc dw_locate(const GroupLds& gl, const Space& sp, int tile_id) {
  const int per = sp.MBt * sp.NBt;   // tiles of one group
  const int p = tile_id / per, local = tile_id % per;
  DwLoc d;
  d.g = gl.ord[p];
  const int band = GM_BAND * sp.NBt;
  const int sup = local / band, within = local % band;
  const int first = sup * GM_BAND;
  const int gsz = min(GM_BAND, sp.MBt - first);
  d.m0 = (first + within % gsz) * BM;
  d.n0 = (within / gsz) * BN;
  d.rows0 = gl.lo[d.g];
  d.kdim = gl.hi[d.g] - gl.lo[d.g];
  return d;
}
// P and Q views of a weight-gradient tile (rows not gathered): the group's
// K rows of X and of W (arows: the rows P can touch)
template <typename T>
__device__ __forceinline__ void dw_views(const GmmArgs& a, const DwLoc& d, int arows, View& va,
                                         View& vb) {
  constexpr int ES = Cfg<T>::ES;
  const bool sh = d.g >= a.G;
  const long long xg = a.dense ? (long long)d.g * a.x_gs * ES : 0;
  const void* pb = sh ? a.sX : (const void*)((const char*)a.X + xg);
  const void* qb =
      sh ? a.sW : (const void*)((const char*)a.W + (a.dense ? (long long)d.g * a.w_gs * ES : 0));
  va = make_view((const char*)pb + (long long)d.rows0 * a.ldx * ES, (long long)arows * a.ldx * ES,
                 a.ldx, a.M);
  vb = make_view((const char*)qb + (long long)d.rows0 * a.ldw * ES, (long long)d.kdim * a.ldw * ES,
                 a.ldw, a.N);
}

// Weight-gradient tiles overlap across tiles (bf16, 4 waves, rows not
// gathered, bf16 output, one K step per A step): while a tile's epilogue
// runs, the next tile's first two K steps are already being copied into
// ring slots 2-3, and the epilogue stages its output through slots 0-1 in
// two bf16 slices of 128 columns, so the copies are issued ahead of the
// epilogue's stores and do not wait for them to drain (the vector-memory
// counter retires in issue order).  A prefetched tile runs with its K step kt
// in slot (kt + 2) % 4.  DW_STORES: buffer stores each thread issues in that
// epilogue (2 slices x 16 chunks), which the prefetched tile's first waits
// allow to be outstanding.
constexpr int DW_STORES = 32;
constexpr int DW_PRE = 2;   // K steps a weight-gradient tile's epilogue copies for the next
__device__ __forceinline__ bool dw_overlap_ok(const GmmArgs& a) {
  return !a.out_f32 && a.krep <= 1;
}
// Copies of K steps 0-1 of weight-gradient tile tile_id into slots 2-3, in
// the order the tile's own prologue would issue them (every K step: the
// DPO P copies, then the DPO Q copies; steps past the last through an empty
// descriptor).
template <typename T, int W>
__device__ __forceinline__ void dw_prefetch(const GmmArgs& a, const GroupLds& gl, const Space& sp,
                                            int tile_id, char* smem) {
  constexpr int ES = Cfg<T>::ES, BK = Cfg<T>::BK, OPB = Cfg<T>::OPB, STAGE_BYTES = 2 * OPB;
  constexpr int DPO = DPO_OF<T, W>;
  DwLoc d = dw_locate(gl, sp, tile_id);
  d.g = uniform(d.g); d.m0 = uniform(d.m0); d.n0 = uniform(d.n0);
  d.rows0 = uniform(d.rows0); d.kdim = uniform(d.kdim);
  View va, vb;
  dw_views<T>(a, d, d.kdim, va, vb);
  uint32_t offa[DPO], offb[DPO];
  mnmajor_offsets<T>(va, d.m0, offa);
  mnmajor_offsets<T>(vb, d.n0, offb);
  const int KT = (d.kdim + BK - 1) / BK;
  const int sa = va.ld * BK * ES, sb = vb.ld * BK * ES;
  const i32x4 rs_none = {0, 0, 0, MOE_RSRC_DW3};
  const uint32_t lds_wa = lds_addr(smem) + (threadIdx.x >> 6) * DPO * 1024;
  const uint32_t lds_wb = lds_addr(smem) + OPB + (threadIdx.x >> 6) * DPO * 1024;
#pragma unroll
  for (int kt = 0; kt < DW_PRE; ++kt) {
    const uint32_t so = (uint32_t)((kt + DW_PRE) * STAGE_BYTES);
#pragma unroll
    for (int j = 0; j < DPO; ++j)
      dma16(kt < KT ? va.rs : rs_none, lds_wa + so + j * 1024, offa[j], kt * sa);
#pragma unroll
    for (int j = 0; j < DPO; ++j)
      dma16(kt < KT ? vb.rs : rs_none, lds_wb + so + j * 1024, offb[j], kt * sb);
  }
}
struct NoPrefetch {
  __device__ void operator()() const {}
};

// Tile tile_id of a product: main loop over K and epilogue.  smem is the
// 128 KB operand ring (also the epilogue's staging), g_idx the gathered-row
// index ring.  drained() runs once per tile, by every thread, at the point
// where every copy of the tile and the scheduler's draw have landed.
template <typename T, int MODE, bool GATHER, bool LIGHT, bool LEAN, int W, bool ACT_DEV = false,
          int WM = 2, bool DEEP = false, typename Drained, typename Prefetch = NoPrefetch>
__device__ __forceinline__ void run_tile(const GmmArgs& a, const GroupLds& gl, const Space& sp,
                                         int tile_id, char* smem, int* g_idx, Drained&& drained,
                                         int pre_in = 0, Prefetch&& prefetch = Prefetch()) {
  using WS = Waves<W, WM>;
  constexpr int NT = WS::NT, WN = WS::WN, FN = WS::FN, HW = WS::HW, BMT = WS::BMT;
  constexpr int ES = Cfg<T>::ES, BK = Cfg<T>::BK;
  // DW with gathered Q rows: the rows change every K step, so each wave also
  // copies its K rows' indices into an LDS ring, two steps before the copies
  // that use them -- one more buffer load per wave per step (GI)
  constexpr bool GLOOP = GATHER && MODE == DW;
  constexpr int GI = GLOOP ? 1 : 0;
  static_assert(!GATHER || MODE == FWD1 || MODE == DW, "rows are gathered in FWD1 and DW");
  static_assert(!LIGHT || (MODE != DW && sizeof(T) == 2), "light builds: bf16 row-tiled modes");
  static_assert(!GLOOP || sizeof(T) == 2, "gathered DW is built for bf16");
  static_assert(W == 4 || (W == 8 && sizeof(T) == 2 && !GLOOP),
                "8 waves: bf16, without the gathered weight-gradient index ring");
  constexpr bool A_MN = (MODE == DW);
  constexpr bool B_MN = (MODE == DX1 || MODE == DX2 || MODE == DW);
  // DEEP (light builds, tiles of at most 64 rows): a stage holds only the
  // A tile's first 64 rows (4 KB) beside the 16 KB B tile, so six stages fit
  // the ring and five K steps are in flight instead of three.  Such a tile
  // is bound by the latency of its weight stream (its few MFMAs and the
  // copies of its padding rows are not what limits it), so more bytes in
  // flight per CU is what speeds it up.  OPB: byte offset of the B tile in
  // a stage.
  static_assert(!DEEP || (LIGHT && WM == 2 && W == 4), "deep ring: light builds, 4 waves");
  // weight-gradient tiles that overlap across tiles (see dw_prefetch)
  constexpr bool PF = MODE == DW && sizeof(T) == 2 && !GLOOP && W == 4 && WM == 2 && !DEEP;
  constexpr int STAGES = DEEP ? 6 : Cfg<T>::STAGES;
  constexpr int OPB = DEEP ? 4096 : Cfg<T>::OPB;
  constexpr int STAGE_BYTES = OPB + Cfg<T>::OPB;
  static_assert(WM == 2 || (WM == 1 && W == 4 && sizeof(T) == 2 && MODE != DW && !LIGHT),
                "strip tiles: bf16 row-tiled products, 4 waves");
  // buffer loads per wave per K step: DPA for the A tile (BMT rows; DEEP: 64),
  // DPB for the B tile (256 rows or columns)
  constexpr int DPB = DPO_OF<T, W>;
  constexpr int DPA = DEEP ? 1 : DPB * WM / 2;
  constexpr int DMA_PER_STEP = DPA + DPB;
  // MFMA slots of a half K step that issue the A (first half) and B (second
  // half) copies: right after the fragment loads, or the last slots where
  // a half step has fewer MFMAs than loads and copies
  constexpr int CS1 = (FM + FN < FM * FN - DPA) ? FM + FN : FM * FN - DPA;
  constexpr int CS2 = (FM + FN < FM * FN - DPB) ? FM + FN : FM * FN - DPB;
  static_assert(STAGES * STAGE_BYTES <= RING_BYTES, "stage ring size");
  static_assert(BM * EP_PITCH * 4 <= RING_BYTES, "epilogue slice must fit the ring");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;   // WM x WN wave grid
  const int ng = a.G + a.shared;
  // ---- locate the tile
  int g, m0, n0, rows0 = 0, rows = 0, kdim;
  if constexpr (MODE != DW) {
    const RowTile rt = locate_row_tile(gl, sp, ng, tile_id);
    g = rt.g;
    rows0 = rt.rows0;
    rows = rt.rows;
    m0 = 0;
    n0 = rt.nbi * ((MODE == FWD1) ? BN / 2 : BN);
    kdim = a.K;
  } else {
    const DwLoc d = dw_locate(gl, sp, tile_id);
    g = d.g;
    m0 = d.m0;
    n0 = d.n0;
    rows0 = d.rows0;
    kdim = d.kdim;
  }
  g = uniform(g); m0 = uniform(m0); n0 = uniform(n0);
  rows0 = uniform(rows0); rows = uniform(rows); kdim = uniform(kdim);
  const bool sh = g >= a.G;
  const bool gat = GATHER && !sh;   // routed tile of a gathering launch
  const long long xg = a.dense ? (long long)g * a.x_gs * ES : 0;   // dense group bases
  const int krep = a.krep > 1 ? a.krep : 1;
  const int arows = kdim / krep;   // A rows a DW tile can touch

  // ---- operand views
  View va, vb;
  if constexpr (MODE != DW) {
    const void* xb = sh ? a.sX : (const void*)((const char*)a.X + xg);
    if (gat)   // FWD1: the rows are gathered from the whole token matrix
      va = make_view(a.X, (long long)a.gather_rows * a.ldx * ES, a.ldx, rows);
    else
      va = make_view((const char*)xb + (long long)rows0 * a.ldx * ES,
                     (long long)rows * a.ldx * ES, a.ldx, rows);
    const void* wb = sh ? a.sW : (const void*)((const char*)a.W + (long long)g * a.w_gs * ES);
    const int wrows = (MODE == FWD1) ? 2 * a.I : (B_MN ? a.K : a.N);  // stored rows of W
    const int wcols = B_MN ? a.N : a.K;
    vb = make_view(wb, (long long)wrows * wcols * ES, a.ldw, a.N);
  } else {
    dw_views<T>(a, DwLoc{g, m0, n0, rows0, kdim}, arows, va, vb);
    if (gat)   // DW: Q's K rows are gathered from the whole token matrix
      vb = make_view(a.W, (long long)a.gather_rows * a.ldw * ES, a.ldw, a.N);
  }
  // a weight-gradient tile whose first K steps the previous tile's epilogue
  // copied (slots 2-3): its K step kt lives in slot (kt + 2) % 4
  const bool pf_ok = PF && dw_overlap_ok(a);
  const int pre = uniform((PF && pre_in) ? DW_PRE : 0);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = (kdim + BK - 1) / BK;   // K steps with data
  uint32_t offa[DPA], offb[DPB];
  if constexpr (A_MN) mnmajor_offsets<T>(va, m0, offa);
  else if (GATHER && MODE == FWD1 && gat)
    kmajor_offsets_gather<T>(va, a.gather, rows0, rows, offa);
  else kmajor_offsets<T, false, WS::WTN>(va, m0, 0, offa);
  if constexpr (GLOOP) {
    // gathered Q: only the column part is fixed; the row part comes with
    // each K step's indices (view with ld 0 gives column offsets)
    View vc = vb;
    if (gat) vc.ld = 0;
    mnmajor_offsets<T>(vc, n0, offb);
  } else if constexpr (B_MN) mnmajor_offsets<T>(vb, n0, offb);
  else kmajor_offsets<T, MODE == FWD1, WS::WTN>(vb, n0, a.I, offb);
  const int sa = A_MN ? va.ld * BK * ES : BK * ES;   // uniform offset per K step
  const int sb = (GLOOP && gat) ? 0 : (B_MN ? vb.ld * BK * ES : BK * ES);
  auto issue = [&](int kt) {
    const char* st = smem + (kt % STAGES) * STAGE_BYTES;
    issue_op(va, st, offa, (kt / krep) * sa);
    issue_op(vb, st + OPB, offb, kt * sb);
  };
  // copy j of K step kt (j < DPA: operand A, else B); a step past the
  // last one copies through an empty descriptor, which moves no HBM bytes
  // and only writes zeros into a stage nobody reads
  const i32x4 rs_none = {0, 0, 0, MOE_RSRC_DW3};
  const uint32_t lds_wa = lds_addr(smem) + (threadIdx.x >> 6) * DPA * 1024;
  const uint32_t lds_wb = lds_addr(smem) + OPB + (threadIdx.x >> 6) * DPB * 1024;
  // (the A step index is kt / krep; ka_next tracks it for the next step to
  // issue, ka_rep the steps already issued from that A step)
  int ka_next = pre, ka_rep = 0;   // (prefetched: steps 0 .. pre-1 issued)
  auto issue1 = [&](int kt, int j) {
    const uint32_t so = (uint32_t)(((kt + pre) % STAGES) * STAGE_BYTES);
    const bool live = kt < KT;
    if (j < DPA)
      dma16(live ? va.rs : rs_none, lds_wa + so + j * 1024, offa[j], ka_next * sa);
    else
      dma16(live ? vb.rs : rs_none, lds_wb + so + (j - DPA) * 1024, offb[j - DPA], kt * sb);
    if (j == DMA_PER_STEP - 1 && ++ka_rep == krep) { ka_rep = 0; ++ka_next; }
  };
  auto stage = [&](int kt) { return (const char*)smem + ((kt + pre) % STAGES) * STAGE_BYTES; };
  // GLOOP: B copy j of a step covers K rows 8 wave + 2 j + (0, 1), lane l
  // the row l / 32.  The indices of a wave's 8 rows of step kt are copied
  // to its slot kt % 4 in the order 0 2 4 6 1 3 5 7, so a lane's four
  // indices are one 16-byte read.
  const int hrow = lane >> 5;
  i32x4 rs_g = rs_none;
  uint32_t goff = OOB;
  if constexpr (GLOOP) {
    if (gat)
      rs_g = raw_rsrc((const char*)a.gather + (long long)rows0 * 4,
                      clamp_bytes((long long)kdim * 4));
    goff = lane < 8 ? (uint32_t)((8 * wave + 2 * (lane & 3) + (lane >> 2)) * 4) : OOB;
  }
  const uint32_t lds_g = lds_addr((const char*)g_idx) + (uint32_t)(wave * 4 * 256);
  const uint32_t rowb = (uint32_t)(vb.ld * ES);
  auto issue_idx = [&](int kt) {
    dma4(kt < KT ? rs_g : rs_none, lds_g + (uint32_t)((kt & 3) * 256), goff, kt * BK * 4);
  };
  auto read_idx = [&](int kt) {
    return *(const u32x4*)(g_idx + (wave * 4 + (kt & 3)) * 64 + 4 * hrow);
  };
  auto issue_b = [&](int kt, int j, const u32x4& iv) {
    const uint32_t so = (uint32_t)((kt % STAGES) * STAGE_BYTES);
    const int krow = kt * BK + 8 * wave + 2 * j + hrow;
    const uint32_t vo =
        gat ? ((krow < kdim && offb[j] != OOB) ? iv[j] * rowb + offb[j] : OOB) : offb[j];
    dma16(kt < KT ? vb.rs : rs_none, lds_wb + so + j * 1024, vo, kt * sb);
    if (j == DPB - 1 && ++ka_rep == krep) { ka_rep = 0; ++ka_next; }
  };

  if (KT > 0) {
    if constexpr (sizeof(T) == 2) {
      // steps 0 .. STAGES-2 in flight (empty copies past the end), so the
      // wait counts below hold for every K step
      if constexpr (GLOOP) {
        // indices of steps 0-2 first; then per step A, B and the indices
        // of two steps on, in the order the loop keeps
        issue_idx(0);
        issue_idx(1);
        issue_idx(2);
        wait_vm<0>();
        asm volatile("" ::: "memory");
        const u32x4 iv[3] = {read_idx(0), read_idx(1), read_idx(2)};
#pragma unroll
        for (int kt = 0; kt < STAGES - 1; ++kt) {
#pragma unroll
          for (int j = 0; j < DPA; ++j) issue1(kt, j);
#pragma unroll
          for (int j = 0; j < DPB; ++j) issue_b(kt, j, iv[kt]);
          if (kt >= 1) issue_idx(kt + 2);
        }
      } else {
#pragma unroll
        for (int kt = 0; kt < STAGES - 1; ++kt)
          if (kt >= pre)
#pragma unroll
            for (int j = 0; j < DMA_PER_STEP; ++j) issue1(kt, j);
      }
      // (prefetched: the previous tile's epilogue stores were issued after
      // steps 0-1, so they may still be outstanding here)
      if constexpr (PF) {
        if (pre) wait_vm<(STAGES - 2) * DMA_PER_STEP + DW_STORES>();
        else wait_vm<(STAGES - 2) * DMA_PER_STEP>();
      } else {
        wait_vm<(STAGES - 2) * DMA_PER_STEP + 2 * GI>();
      }
    } else {
      for (int kt = 0; kt < STAGES - 1 && kt < KT; ++kt) issue(kt);
      if (KT >= 3) wait_vm<2 * DMA_PER_STEP>();
      else if (KT == 2) wait_vm<DMA_PER_STEP>();
      else wait_vm<0>();
    }
    __syncthreads();
    if constexpr (sizeof(T) == 2) {
      // two fragment sets in ping-pong.  Each half K step's 16 MFMAs carry
      // the other work woven between them (pinned by scheduling barriers),
      // so the matrix pipe never waits on a burst of LDS reads or copy
      // issues: the first half loads the second half's fragments and issues
      // the A copies of step kt+3; the second half (after the barrier)
      // loads the first half fragments of step kt+1 and issues the B copies
      // of step kt+3 (step kt+3's stage held step kt-1, whose last reads
      // retired at the previous barrier; splitting a step's copies over two
      // halves measured ~10% fewer cycles per step than issuing them
      // together).  Steps past the end
      // copy through the empty descriptor, so every step looks the same.
      // LIGHT builds: the loop is built per count FA of this wave's A
      // fragments that hold rows of the tile; in a tile of a group with few
      // rows the upper fragments (and the lower waves) see padding only, so
      // their MFMAs and A-fragment reads are left out (their accumulators
      // stay zero and their rows are never stored).  Copies, waits and
      // barriers are the same in every build, so the waves of a workgroup
      // stay in step, and every output is the same bits as without.
      auto kloop = [&](auto fa_c) {
        constexpr int FA = decltype(fa_c)::value;
        // fragment q of a load (q < FM: A fragment q, else B fragment q - FM)
        auto need = [](int q) { return q < FM ? q < FA : FA > 0; };
        Frags<T, A_MN, B_MN, W, WM> f0, f1;
#pragma unroll
        for (int q = 0; q < FM + FN; ++q)
          if (need(q)) f0.load1(stage(0), stage(0) + OPB, wm, wn, 0, q);
        for (int kt = 0; kt < KT; ++kt) {
          const char* cs = stage(kt);
          const char* ns = stage(kt + 1);
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int q = i * FN + j;
              if (i < FA) acc[i][j] = mfma_step(f0.b[j], f0.a[i], acc[i][j]);
              __builtin_amdgcn_sched_barrier(0);
              if (q < FM + FN && need(q)) f1.load1(cs, cs + OPB, wm, wn, 1, q);
              if (q >= CS1 && q - CS1 < DPA) issue1(kt + STAGES - 1, q - CS1);
              __builtin_amdgcn_sched_barrier(0);
            }
          wait_vm<(STAGES - 3) * DMA_PER_STEP + DPA + GI>();
          __syncthreads();
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int q = i * FN + j;
              if (i < FA) acc[i][j] = mfma_step(f1.b[j], f1.a[i], acc[i][j]);
              __builtin_amdgcn_sched_barrier(0);
              if (q < FM + FN && need(q)) f0.load1(ns, ns + OPB, wm, wn, 0, q);
              if (q >= CS2 && q - CS2 < DPB) issue1(kt + STAGES - 1, DPA + q - CS2);
              __builtin_amdgcn_sched_barrier(0);
            }
        }
      };
      if constexpr (DEEP) {
        // at most 64 rows: the upper waves hold padding only, the lower ones
        // one or two fragments of rows
        const int rw = rows - wm * WTM;
        const int fa = uniform(rw <= 0 ? 0 : min(2, (rw + 31) / 32));
        switch (fa) {
          case 0: kloop(std::integral_constant<int, 0>{}); break;
          case 1: kloop(std::integral_constant<int, 1>{}); break;
          default: kloop(std::integral_constant<int, 2>{}); break;
        }
      } else if constexpr (LIGHT) {
        const int rw = rows - wm * WTM;             // rows of the tile in this wave's half
        const int fa = sp.light ? uniform(rw <= 0 ? 0 : min(FM, (rw + 31) / 32)) : FM;
        switch (fa) {
          case 0: kloop(std::integral_constant<int, 0>{}); break;
          case 1: kloop(std::integral_constant<int, 1>{}); break;
          case 2: kloop(std::integral_constant<int, 2>{}); break;
          case 3: kloop(std::integral_constant<int, 3>{}); break;
          default: kloop(std::integral_constant<int, FM>{}); break;
        }
      } else {
        Frags<T, A_MN, B_MN, W, WM> f0, f1;
        f0.load(stage(0), stage(0) + OPB, wm, wn, 0);
        for (int kt = 0; kt < KT; ++kt) {
          const char* cs = stage(kt);
          const char* ns = stage(kt + 1);
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int q = i * FN + j;
              acc[i][j] = mfma_step(f0.b[j], f0.a[i], acc[i][j]);
              __builtin_amdgcn_sched_barrier(0);
              if (q < FM + FN) f1.load1(cs, cs + OPB, wm, wn, 1, q);
              if (q >= CS1 && q - CS1 < DPA) issue1(kt + STAGES - 1, q - CS1);
              __builtin_amdgcn_sched_barrier(0);
            }
          // K step kt+1 has landed once at most the copies issued after it
          // (steps kt+2 .. kt+STAGES-2, and step kt+STAGES-1's A copies) are
          // outstanding; the barrier extends that to all waves and retires
          // every read of the stage refilled next
          // (GLOOP: also step kt+3's indices, issued right after step
          // kt+1's B copies, and one index copy more per step since)
          // (prefetched tile, step 0: the previous tile's epilogue stores,
          // issued after step 1, may still be outstanding)
          if constexpr (PF) {
            if (pre && kt == 0) wait_vm<(STAGES - 3) * DMA_PER_STEP + DPA + DW_STORES>();
            else wait_vm<(STAGES - 3) * DMA_PER_STEP + DPA>();
          } else {
            wait_vm<(STAGES - 3) * DMA_PER_STEP + DPA + GI>();
          }
          __syncthreads();
          u32x4 ivn;
          if constexpr (GLOOP) ivn = read_idx(kt + STAGES - 1);
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int q = i * FN + j;
              acc[i][j] = mfma_step(f1.b[j], f1.a[i], acc[i][j]);
              __builtin_amdgcn_sched_barrier(0);
              if (q < FM + FN) f0.load1(ns, ns + OPB, wm, wn, 0, q);
              if (q >= CS2 && q - CS2 < DPB) {
                if constexpr (GLOOP) issue_b(kt + STAGES - 1, q - CS2, ivn);
                else issue1(kt + STAGES - 1, DPA + q - CS2);
              } else if (GLOOP && q == CS2 + DPB) {
                issue_idx(kt + STAGES + 1);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
        }
      }
    } else {
      Frags<T, A_MN, B_MN, W, WM> cur, nxt;
      cur.load(stage(0), stage(0) + OPB, wm, wn, 0);
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int ks = 0; ks < Cfg<T>::KS; ++ks) {
          if (ks == Cfg<T>::KS - 1) {
            if (kt + 1 < KT) {
              if (kt + 2 < KT) wait_vm<DMA_PER_STEP>();
              else wait_vm<0>();
              __syncthreads();
              if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1);
              nxt.load(stage(kt + 1), stage(kt + 1) + OPB, wm, wn, 0);
            }
          } else {
            nxt.load(stage(kt), stage(kt) + OPB, wm, wn, ks + 1);
          }
          cur.mma(acc);
          cur = nxt;
        }
      }
    }
  }

  // ---- epilogue: the tile leaves through LDS in 256 x 128 fp32 slices, so
  // every HBM access is a 16-byte row chunk.  Slice s holds fragments 2s and
  // 2s+1 of every wave (FWD1: s = 0 gate, s = 1 up columns).
  // a per-tile copy of the thread index: the epilogue's address arithmetic
  // then belongs to this tile and is not kept live (and spilled) across
  // the persistent loop as an invariant
  int etid = threadIdx.x;
  asm volatile("" : "+v"(etid));
  const int elane = etid & 63;
  wait_vm<0>();      // the empty copies past the last step (and the draw) have landed
  drained();   // the scheduler's draw has returned: publish the next tile
  __syncthreads();   // every wave is done with the ring
  if constexpr (PF) {
    if (pf_ok) {
      // the next tile's first K steps into slots 2-3 (if it is a weight-
      // gradient tile of this launch), ahead of this tile's stores
      prefetch();
      // the output leaves through slots 0-1 in two bf16 slices: slice h
      // holds fragments 2h and 2h+1 of every wave, LDS column c (of 128) =
      // wn * 64 + the column in those two fragments, i.e. tile column
      // wn * WTN + 64 h + c % 64; 16-byte unit u of row r sits at u ^ (r & 15)
      // with its two 8-byte halves swapped where bits 3 and 4 of r differ, so
      // the rows of a fragment's write hit distinct banks 16 or 32 lanes at a
      // time.  Rounded to bf16 once, as the plain store rounds.
      const int m = elane & 31;
      void* cb = sh ? a.sC : (void*)((char*)a.C + (long long)g * a.c_gs * ES);
      const __amdgpu_buffer_rsrc_t cr = make_rsrc(cb, out_bytes((long long)a.M * a.ldc * ES));
      char* const sl = smem;
      auto slice2 = [&](auto hc) {
        constexpr int h = decltype(hc)::value;
#pragma unroll
        for (int f = 0; f < FM; ++f)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
              const int row = wm * WTM + f * 32 + m;
              const int c = wn * 64 + j * 32 + rq * 8 + (elane >> 5) * 4;
              // (the empty asm keeps each conversion at its store: converted
              // ahead of time, the whole tile's bf16 values would not fit the
              // registers)
              float x0 = acc[f][2 * h + j][rq * 4 + 0], x1 = acc[f][2 * h + j][rq * 4 + 1];
              float x2 = acc[f][2 * h + j][rq * 4 + 2], x3 = acc[f][2 * h + j][rq * 4 + 3];
              asm volatile("" : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3));
              u32x2 v;
              v.x = f32_to_bf16(x0) | (f32_to_bf16(x1) << 16);
              v.y = f32_to_bf16(x2) | (f32_to_bf16(x3) << 16);
              *(u32x2*)(sl + row * 256 + (((c >> 3) ^ (row & 15)) << 4) +
                        ((((c >> 2) ^ (row >> 3) ^ (row >> 4)) & 1) * 8)) = v;
            }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 256 * 16 / NT; ++it) {
          const int idx = it * NT + etid;
          const int row = idx >> 4, u = idx & 15;
          u32x4 v = *(const u32x4*)(sl + row * 256 + ((u ^ (row & 15)) << 4));
          if (((row >> 3) ^ (row >> 4)) & 1) v = u32x4{v.z, v.w, v.x, v.y};
          const int n = n0 + (u >> 3) * WS::WTN + 64 * h + (u & 7) * 8;
          const int mm = m0 + row;
          buf_store16_nt(cr, (mm < a.M && n < a.N) ? (uint32_t)(mm * a.ldc + n) * 2u : DROP, v);
        }
        __syncthreads();
      };
      slice2(std::integral_constant<int, 0>{});
      slice2(std::integral_constant<int, 1>{});
      return;
    }
  }
  float* ep = (float*)smem;
  auto put = [&](auto fn0c, auto&& value) {
    // fragments fn0 .. fn0 + FN/2 - 1 of each wave -> LDS columns
    // wn*HW + j*32 + (0..31) (fn0 is a compile-time constant so the
    // accumulators stay in registers); 16-byte granule g of row m sits at
    // g ^ (m % 32), so the 32 rows of a store and the 16 chunks of a row read
    // all hit distinct banks
    constexpr int slice_fn0 = decltype(fn0c)::value;
    const int m = elane & 31;
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int j = 0; j < FN / 2; ++j)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int row = wm * WTM + f * 32 + m;
          const int g = (wn * HW + j * 32 + rq * 8 + (elane >> 5) * 4) >> 2;
          f32x4 v;
          v.x = value(f, slice_fn0 + j, rq * 4 + 0);
          v.y = value(f, slice_fn0 + j, rq * 4 + 1);
          v.z = value(f, slice_fn0 + j, rq * 4 + 2);
          v.w = value(f, slice_fn0 + j, rq * 4 + 3);
          *(f32x4*)(ep + row * EP_PITCH + ((g ^ m) << 2)) = v;
        }
    __syncthreads();
  };
  auto take = [&](auto&& consume) {
    // BMT rows x 16 chunks of 8 columns, BMT * 16 / NT per thread
#pragma unroll 4
    for (int it = 0; it < BMT * 16 / NT; ++it) {
      const int idx = it * NT + etid;
      const int row = idx >> 4, cc = (idx & 15) * 8;
      const int sw = row & 31;
      float v[8];
      const f32x4 lo = *(const f32x4*)(ep + row * EP_PITCH + (((cc >> 2) ^ sw) << 2));
      const f32x4 hi = *(const f32x4*)(ep + row * EP_PITCH + ((((cc >> 2) + 1) ^ sw) << 2));
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
      consume(row, cc, v);
    }
    __syncthreads();
  };
  auto acc_of = [&](int f, int fn, int r) { return acc[f][fn][r]; };

  // slice sl of the finished tile -> consume(row, c, v[8])
  auto emit = [&](auto slc, auto&& consume) {
    constexpr int sl = decltype(slc)::value;
    put(std::integral_constant<int, sl * (FN / 2)>{}, acc_of);
    take(consume);
  };

  // 8 values at element elem of an output (dropped unless ok)
  // every output leaves with the streaming cache policy: measured ~1.5%
  // faster over the layer step than plain stores (also with yp or act kept
  // cached for the kernel that reads them next)
  auto store8 = [&](const __amdgpu_buffer_rsrc_t& rs, bool ok, uint32_t elem, const float* v) {
    if constexpr (sizeof(T) == 2) {
      buf_store16_nt(rs, ok ? elem * 2u : DROP, pack16(v, T()));
    } else {
      buf_store16_nt(rs, ok ? elem * 4u : DROP, pack16(v, T()));
      buf_store16_nt(rs, ok ? elem * 4u + 16u : DROP, pack16(v + 4, T()));
    }
  };
  // act rows another XCD reads within the same launch: stored at device
  // scope, so they are visible everywhere once the stores have completed
  auto store8_dev = [&](const __amdgpu_buffer_rsrc_t& rs, bool ok, uint32_t elem, const float* v) {
    if constexpr (sizeof(T) == 2) {
      buf_store16_dev(rs, ok ? elem * 2u : DROP, pack16(v, T()));
    } else {
      buf_store16_dev(rs, ok ? elem * 4u : DROP, pack16(v, T()));
      buf_store16_dev(rs, ok ? elem * 4u + 16u : DROP, pack16(v + 4, T()));
    }
  };
  // 8 values at element elem of an operand (zeros unless ok)
  auto load8 = [&](const __amdgpu_buffer_rsrc_t& rs, bool ok, uint32_t elem, float* v) {
    if constexpr (sizeof(T) == 2) {
      unpack16(buf_load16(rs, ok ? elem * 2u : OOB), v, T());
    } else {
      unpack16(buf_load16(rs, ok ? elem * 4u : OOB), v, T());
      unpack16(buf_load16(rs, ok ? elem * 4u + 16u : OOB), v + 4, T());
    }
  };
  if constexpr (MODE == FWD1) {
    // fragments 0 .. FN/2-1 of a wave hold gate columns i0 + wn*HW + j*32 +
    // elane%32, fragments FN/2 .. FN-1 the matching up columns; LDS column c
    // is i = i0 + c
    void* hb = sh ? a.sC : a.C;
    void* ab = sh ? a.sC2 : a.C2;
    const __amdgpu_buffer_rsrc_t hr = make_rsrc((char*)hb + (long long)rows0 * a.ldc * ES,
                                                out_bytes((long long)rows * a.ldc * ES));
    const __amdgpu_buffer_rsrc_t ar = make_rsrc((char*)ab + (long long)rows0 * a.ldc2 * ES,
                                                out_bytes((long long)rows * a.ldc2 * ES));
    auto store_gate = [&](int row, int c, const float* v) {
      store8(hr, row < rows && n0 + c < a.I, (uint32_t)(row * a.ldc + n0 + c), v);
    };
    auto store_up = [&](int row, int c, const float* v) {
      store8(hr, row < rows && n0 + c < a.I, (uint32_t)(row * a.ldc + a.I + n0 + c), v);
    };
    auto store_act = [&](int row, int c, const float* v) {
      if constexpr (ACT_DEV)
        store8_dev(ar, row < rows && n0 + c < a.I, (uint32_t)(row * a.ldc2 + n0 + c), v);
      else
        store8(ar, row < rows && n0 + c < a.I, (uint32_t)(row * a.ldc2 + n0 + c), v);
    };
    // gate slice out; then act = silu(g) * u replaces it in LDS (each
    // elane rewrites the very words it put, so no barrier in between and
    // the gate accumulators are dead once the slice is staged); up last
    put(std::integral_constant<int, 0>{}, acc_of);
    take(store_gate);
    {
      const int m = elane & 31;
#pragma unroll
      for (int f = 0; f < FM; ++f)
#pragma unroll
        for (int j = 0; j < FN / 2; ++j)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int row = wm * WTM + f * 32 + m;
            const int g = (wn * HW + j * 32 + rq * 8 + (elane >> 5) * 4) >> 2;
            f32x4* pp = (f32x4*)(ep + row * EP_PITCH + ((g ^ m) << 2));
            f32x4 v = *pp;
            constexpr int U = FN / 2;
            const f32x4 u = {acc[f][U + j][rq * 4 + 0], acc[f][U + j][rq * 4 + 1],
                             acc[f][U + j][rq * 4 + 2], acc[f][U + j][rq * 4 + 3]};
            v.x = swiglu_act<T>(v.x, u.x);
            v.y = swiglu_act<T>(v.y, u.y);
            v.z = swiglu_act<T>(v.z, u.z);
            v.w = swiglu_act<T>(v.w, u.w);
            *pp = v;
          }
      __syncthreads();
    }
    take(store_act);
    put(std::integral_constant<int, FN / 2>{}, acc_of);
    take(store_up);
  } else {
    // LDS column c of slice h is tile column (c/HW)*WTN + HW h + c%HW
    auto slice = [&](auto hc) {
      constexpr int h = decltype(hc)::value;
      if constexpr (MODE == DX1) {
        const void* hb = sh ? a.sAux : a.aux;
        void* db = sh ? a.sC : a.C;
        const __amdgpu_buffer_rsrc_t hr = make_rsrc(
            (const char*)hb + (long long)rows0 * a.ldaux * ES, clamp_bytes((long long)rows * a.ldaux * ES));
        const __amdgpu_buffer_rsrc_t dr = make_rsrc(
            (char*)db + (long long)rows0 * a.ldc * ES, out_bytes((long long)rows * a.ldc * ES));
        // d(act) -> d(gate), d(up) of act = silu(gate) * up
        auto bwd8 = [&](bool ok, int row, int i, const float* d, const float* gv,
                        const float* uv) {
          float dg[8], du[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float sg = sigmoidf_(gv[e]);
            dg[e] = d[e] * uv[e] * sg * (1.0f + gv[e] * (1.0f - sg));
            du[e] = d[e] * gv[e] * sg;
          }
          store8(dr, ok, (uint32_t)(row * a.ldc + i), dg);
          store8(dr, ok, (uint32_t)(row * a.ldc + a.I + i), du);
        };
        if (sizeof(T) == 2) {
          // bf16: the slice's gate/up chunks (BMT * 16 / NT per thread) are
          // requested before the accumulators are staged, so their latency
          // hides behind the LDS round trip instead of serializing with the
          // stores (a load may not pass an earlier store to a buffer that
          // could alias).  LEAN builds hold 8 chunks at a time (the second
          // half is requested after the first half's stores), which keeps a
          // kernel that also holds another product's code within the
          // register file
          constexpr int CH = BMT * 16 / NT;      // chunks per thread
          constexpr int PF = LEAN ? CH / 2 : CH;
          u32x4 graw[PF], uraw[PF];
          auto fetch = [&](int it) {
            const int idx = it * NT + etid;
            const int row = idx >> 4, cc = (idx & 15) * 8;
            const int i = n0 + (cc / HW) * (2 * HW) + HW * h + (cc % HW);
            const bool ok = row < rows && i < a.I;
            graw[it % PF] = buf_load16(hr, ok ? (uint32_t)(row * a.ldaux + i) * 2u : OOB);
            uraw[it % PF] = buf_load16(hr, ok ? (uint32_t)(row * a.ldaux + a.I + i) * 2u : OOB);
          };
          auto finish = [&](int it) {
            const int idx = it * NT + etid;
            const int row = idx >> 4, cc = (idx & 15) * 8;
            const int sw = row & 31;
            const f32x4 lo = *(const f32x4*)(ep + row * EP_PITCH + (((cc >> 2) ^ sw) << 2));
            const f32x4 hi = *(const f32x4*)(ep + row * EP_PITCH + ((((cc >> 2) + 1) ^ sw) << 2));
            const float d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            const int i = n0 + (cc / HW) * (2 * HW) + HW * h + (cc % HW);
            float gv[8], uv[8];
            unpack16(graw[it % PF], gv, T());
            unpack16(uraw[it % PF], uv, T());
            bwd8(row < rows && i < a.I, row, i, d, gv, uv);
          };
          // first half requested before the staging, second half after it
          // (ahead of the first half's stores; LEAN: after them)
#pragma unroll
          for (int it = 0; it < CH / 2; ++it) fetch(it);
          put(std::integral_constant<int, h * (FN / 2)>{}, acc_of);
          if constexpr (LEAN) {
#pragma unroll
            for (int it = 0; it < CH / 2; ++it) finish(it);
#pragma unroll
            for (int it = CH / 2; it < CH; ++it) fetch(it);
#pragma unroll
            for (int it = CH / 2; it < CH; ++it) finish(it);
          } else {
#pragma unroll
            for (int it = CH / 2; it < CH; ++it) fetch(it);
#pragma unroll
            for (int it = 0; it < CH; ++it) finish(it);
          }
          __syncthreads();
        } else {
          emit(hc, [&](int row, int c, const float* d) {
            const int i = n0 + (c / HW) * (2 * HW) + HW * h + (c % HW);
            const bool ok = row < rows && i < a.I;
            float gv[8], uv[8];
            load8(hr, ok, (uint32_t)(row * a.ldaux + i), gv);
            load8(hr, ok, (uint32_t)(row * a.ldaux + a.I + i), uv);
            bwd8(ok, row, i, d, gv, uv);
          });
        }
      } else {
        // plain store: FWD2 / DX2 rows of C, or DW: dW[g] (M x N)
        void* cb;
        long long cbytes;
        int lim_m;
        const int OS = a.out_f32 ? 4 : ES;   // bytes per output element
        if constexpr (MODE == DW) {
          cb = sh ? a.sC : (void*)((char*)a.C + (long long)g * a.c_gs * OS);
          cbytes = (long long)a.M * a.ldc * OS;
          lim_m = a.M;
        } else {
          cb = (char*)(sh ? a.sC : a.C) + (a.dense ? (long long)g * a.c_gs * OS : 0) +
               (long long)rows0 * a.ldc * OS;
          cbytes = (long long)rows * a.ldc * OS;
          lim_m = rows;
        }
        const __amdgpu_buffer_rsrc_t cr = make_rsrc(cb, out_bytes(cbytes));
        // (the output type is chosen outside the loop, which then
        // unrolls into batches of LDS reads and stores)
        auto place = [&](int row, int c, bool& ok) {
          const int n = n0 + (c / HW) * (2 * HW) + HW * h + (c % HW);
          const int m = m0 + row;
          ok = m < lim_m && n < a.N;
          return (uint32_t)(m * a.ldc + n);
        };
        if (a.out_f32) {
          emit(hc, [&](int row, int c, const float* v) {
            bool ok;
            const uint32_t e = place(row, c, ok);
            buf_store16_nt(cr, ok ? e * 4u : DROP, pack16(v, 0.0f));
            buf_store16_nt(cr, ok ? e * 4u + 16u : DROP, pack16(v + 4, 0.0f));
          });
        } else {
          emit(hc, [&](int row, int c, const float* v) {
            bool ok;
            const uint32_t e = place(row, c, ok);
            store8(cr, ok, e, v);
          });
        }
      }
    };
    slice(std::integral_constant<int, 0>{});
    slice(std::integral_constant<int, 1>{});
  }
}

// A row tile of at most 128 rows runs as a strip tile (bf16, 4 waves):
// half the copies and MFMAs of a full tile, the same bits.
template <typename T, int MODE, bool GATHER, bool LEAN, int W, bool ACT_DEV = false,
          typename Drained>
__device__ __forceinline__ void run_row_tile(const GmmArgs& a, const GroupLds& gl,
                                             const Space& sp, int tile_id, char* smem,
                                             int* g_idx, Drained&& drained) {
  static_assert(MODE != DW, "row-tiled products");
  if constexpr (sizeof(T) == 2 && W == 4) {
    if (uniform(locate_row_tile(gl, sp, a.G + a.shared, tile_id).rows) <= WTM) {
      // (LEAN: the strip's epilogue holds fewer prefetched chunks, so the
      // kernel that also holds the full tile's code stays in its registers)
      run_tile<T, MODE, GATHER, false, true, W, ACT_DEV, 1>(a, gl, sp, tile_id, smem, g_idx,
                                                           drained);
      return;
    }
  }
  run_tile<T, MODE, GATHER, false, LEAN, W, ACT_DEV, 2>(a, gl, sp, tile_id, smem, g_idx, drained);
}

// ---------------------------------------------------------------- the kernels
// Persistent tile loop.  Tiles are dealt in rounds of one per workgroup; in
// each round the workgroups of XCD x (workgroup i runs on XCD i % 8) take the
// round's x-th block of consecutive tiles, so an XCD's workgroups share
// operand panels in its L2 and the whole chip works on one compact stretch of
// tiles at a time (whose operands stay in the MALL).  Without a workspace
// workgroup w of an XCD takes the w-th tile of each of its blocks; with one
// the XCD's workgroups draw its tiles in order from the XCD's counter, so a
// workgroup that starts late (its CU was still busy with another kernel) or
// drew short tiles just takes fewer or more.  body(n, drained, peek) runs the
// n-th tile of the launch's sequence of total tiles; peek() gives the
// position of the workgroup's next tile (>= total: none) once drained() has
// run and a barrier has followed.
template <typename Body>
__device__ __forceinline__ void persistent_loop(int* ctr, int total, int* s_next, Body&& body) {
  const int tid = threadIdx.x;
  const int nwg = gridDim.x;
  const int bid = blockIdx.x;
  const int nx = (nwg % 8 == 0) ? 8 : 1;
  const int xcd = bid % nx, wpx = nwg / nx, wix = bid / nx;
  // n-th tile of this XCD's sequence
  auto tile_of = [&](int n) { return (n / wpx) * nwg + xcd * wpx + n % wpx; };
  // ctr: [0, 8) per-XCD tile counters, [8] finished workgroups (NULL: static)
  const bool dyn = ctr != nullptr;
  // thread 0, with the workspace: once the sequence of XCD vx (its own at
  // first) is used up, the workgroup goes on drawing from the next XCD's
  // counter, so XCDs that ran short tiles take the unstarted tiles of XCDs
  // still busy with long ones (with a fixed sequence per XCD, the last
  // round's long tiles landed on two XCDs while six others idled up to
  // 170 us); every XCD's first wpx tiles are the static first tiles of its
  // own workgroups
  int vx = xcd;
  auto pos_in = [&](int x, int k) { return (k / wpx) * nwg + x * wpx + k % wpx; };
  auto resolve = [&](int k) {   // position of draw k of XCD vx's counter
    int n = pos_in(vx, wpx + k);
    for (int tries = 1; n >= total && tries < nx; ++tries) {
      vx = (vx + 1) % nx;
      n = pos_in(vx, wpx + __hip_atomic_fetch_add(ctr + vx, 1, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT));
    }
    return n;
  };
  int k = wix;              // static order: index of the tile in the XCD's sequence
  int n = tile_of(k);
  int grab = 0;             // thread 0: the counter value drawn at the start of this tile
  for (bool first = true;; first = false) {
    // every wave is done reading the ring (previous tile) and s_next holds
    // the next tile's position; the previous tile's stores may still be
    // draining -- they overlap this tile's first copies (the copy waits
    // count them too, which only makes them wait longer)
    __syncthreads();
    if (!first) {
      if (dyn) {
        n = *s_next;
      } else {
        k += wpx;
        n = tile_of(k);
      }
    }
    n = uniform(n);
    if (n >= total) break;
    // draw the tile after this one now: the atomic returns long before its
    // value is read, at the epilogue's full wait
    if (dyn && tid == 0)
      grab = __hip_atomic_fetch_add(ctr + vx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    body(
        n,
        [&]() {
          if (dyn && tid == 0) *s_next = resolve(grab);   // read after the next loop-top barrier
        },
        // the next tile's position, once drained() has run and a barrier
        // has followed it (what the next loop top reads)
        [&]() { return uniform(dyn ? *s_next : tile_of(k + wpx)); });
  }
  // every draw of this workgroup has returned (the last one ended the loop);
  // the last workgroup to finish returns the counters to zero for the next call
  if (dyn && tid == 0) {
    const int done = __hip_atomic_fetch_add(ctr + 8, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == nwg - 1)
      for (int i = 0; i <= 8; ++i)
        __hip_atomic_store(ctr + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename T, int MODE, bool GATHER = false, bool LIGHT = false, int W = 4>
__global__ __launch_bounds__(Waves<W>::NT, 1) void gmm_kernel(GmmArgs a) {
  constexpr bool GLOOP = GATHER && MODE == DW;
  constexpr int NT = Waves<W>::NT;
  __shared__ __attribute__((aligned(1024))) char smem[RING_BYTES];
  __shared__ GroupLds gl;
  __shared__ int s_next;
  // GLOOP: [wave][step % 4][64] row indices (lanes 0-7 of each copy carry them)
  __shared__ __attribute__((aligned(16))) int g_idx[GLOOP ? (NT / 64) * 4 * 64 : 4];
  const int ng = a.G + a.shared;
  load_groups(a, gl);
  if constexpr (MODE != DW) tile_prefix(ng, gl);
  else group_order(ng, gl);
  const Space sp = tile_space<MODE, LIGHT>(a, gl, &s_next);
  int pre = 0;   // this workgroup's next tile has its first K steps in the ring
  persistent_loop(a.cnt, sp.total, &s_next, [&](int n, auto&& drained, auto&& peek) {
    if constexpr (MODE != DW && !LIGHT) {   // (DX1 lean: both tile shapes fit the registers)
      run_row_tile<T, MODE, GATHER, MODE == DX1, W>(a, gl, sp, n, smem, g_idx, drained);
    } else if constexpr (LIGHT && W == 4) {
      // light loops in use: a tile of at most 64 rows takes the deep ring
      // (DX1 lean, as above)
      if (sp.light && uniform(locate_row_tile(gl, sp, ng, n).rows) <= 64)
        run_tile<T, MODE, GATHER, true, MODE == DX1, W, false, 2, true>(a, gl, sp, n, smem,
                                                                        g_idx, drained);
      else
        run_tile<T, MODE, GATHER, true, MODE == DX1, W>(a, gl, sp, n, smem, g_idx, drained);
    } else if constexpr (MODE == DW && sizeof(T) == 2 && !GLOOP && W == 4) {
      const int pr = pre;
      pre = 0;
      run_tile<T, MODE, GATHER, LIGHT, false, W>(a, gl, sp, n, smem, g_idx, drained, pr, [&]() {
        const int nn = peek();
        if (nn < sp.total) {
          dw_prefetch<T, W>(a, gl, sp, nn, smem);
          pre = 1;
        }
      });
    } else {
      run_tile<T, MODE, GATHER, LIGHT, false, W>(a, gl, sp, n, smem, g_idx, drained);
    }
  });
}

// Two independent products of one call in one persistent launch (a row-tiled
// product and a weight-gradient product on the same group window), so that
// neither ends in a partial round of its own: the gradient tiles of groups
// whose K (rows) is at least the row-tiled product's K run first, then the
// row-tiled product, then the remaining (short) gradient tiles, which fill
// the last round.
//
// Long tiles (the row-tiled product's and the leading gradient tiles) that
// spill into a last partial round leave most workgroups idle at the end of
// the first launch of a backward call (the short tiles fill only part of
// it), so that launch keeps only as many leading gradient tiles as make its
// long tiles a whole number of rounds; the second launch (a0.M > 0: a0 holds
// the first launch's gradient product) runs the rest first.  Both launches
// derive the split from the same group table, so every tile runs once.

// leading gradient tiles: those of the groups with at least K rows
__device__ __forceinline__ int lead_tiles(const GroupLds& gl, int ng, int K, const Space& s) {
  int lead = 0;
  while (lead < ng && gl.hi[gl.ord[lead]] - gl.lo[gl.ord[lead]] >= K) ++lead;
  return lead * s.MBt * s.NBt;
}
// leading gradient tiles the first launch keeps: n1 row-tiled tiles plus the
// kept ones a multiple of the P workgroups, if dropping at most L gets there
__device__ __forceinline__ int lead_kept(int n1, int L, int P) {
  const int over = (n1 + L) % P;
  return over <= L ? L - over : L;
}

template <typename T, int M1, int M2, int W>
__global__ __launch_bounds__(Waves<W>::NT, 1) void gmm_pair_kernel(GmmArgs a1, GmmArgs a2,
                                                                   GmmArgs a0) {
  static_assert(M1 != DW && M2 == DW, "a row-tiled product and a weight-gradient product");
  __shared__ __attribute__((aligned(1024))) char smem[RING_BYTES];
  __shared__ GroupLds gl;
  __shared__ int s_next;
  __shared__ int g_idx[4];
  const int ng = a1.G + a1.shared;
  load_groups(a1, gl);
  tile_prefix(ng, gl);
  group_order(ng, gl);
  const Space s1 = tile_space<M1, false>(a1, gl, &s_next);
  const Space s2 = tile_space<M2, false>(a2, gl, &s_next);
  const int P = gridDim.x;
  const bool second = a0.M > 0;
  Space s0 = s2;
  // positions: [mv tiles of a0 from tile t0][splitA gradient tiles][row-tiled
  // product][gradient tiles from splitA + skip on]
  int mv = 0, t0 = 0, splitA, skip = 0;
  if (!second) {
    const int L = lead_tiles(gl, ng, a1.K, s2);
    splitA = lead_kept(s1.total, L, P);
    skip = L - splitA;
  } else {
    s0 = tile_space<M2, false>(a0, gl, &s_next);
    // the first launch's row-tiled product had K = a0.M and N = a0.N
    const int n1 = gl.pre[ng] * ((a0.N + BN - 1) / BN);
    const int L = lead_tiles(gl, ng, a0.M, s0);
    t0 = lead_kept(n1, L, P);
    mv = L - t0;
    splitA = lead_tiles(gl, ng, a1.K, s2);
  }
  const int total = mv + s1.total + s2.total - skip;
  int pre = 0;   // this workgroup's next (gradient) tile has its first K steps in the ring
  persistent_loop(a1.cnt, total, &s_next, [&](int n, auto&& drained, auto&& peek) {
    const int p = n - mv;
    if (p >= splitA && p < splitA + s1.total) {
      run_row_tile<T, M1, false, true, W>(a1, gl, s1, p - splitA, smem, g_idx, drained);
    } else {
      const bool f = p < 0;
      const int t = f ? t0 + n : (p < splitA ? p : p - s1.total + skip);
      const int pr = pre;
      pre = 0;
      run_tile<T, M2, false, false, true, W>(
          f ? a0 : a2, gl, f ? s0 : s2, t, smem, g_idx, drained, pr, [&]() {
            if constexpr (sizeof(T) == 2 && W == 4) {
              const int nn = peek();
              const int pp = nn - mv;
              if (nn < total && !(pp >= splitA && pp < splitA + s1.total)) {
                const bool ff = pp < 0;
                const int tt = ff ? t0 + nn : (pp < splitA ? pp : pp - s1.total + skip);
                dw_prefetch<T, W>(ff ? a0 : a2, gl, ff ? s0 : s2, tt, smem);
                pre = 1;
              }
            }
          });
    }
  });
}

// ---------------------------------------------------------------- forward chain
// Both forward products in one persistent launch: every gate/up tile first,
// then the act . W2^T tiles, each of which starts once every gate/up tile
// of its row tile has stored its act rows.  The second product's first
// tiles fill the round the first product leaves partly idle, and the
// launch ends in one tail of short second-product tiles instead of two.
// (Interleaving the products band by band was measured slower: a
// second-product tile claimed one band after its row tile's first-product
// tiles waited ~50 us for them on the Pangu share, as first-product tiles
// are ~4x longer.)  The workgroups of each XCD take positions of this order
// from their XCD's counter, in the same chunks as the single-product
// launches (so an XCD's workgroups share operand panels in its L2).
//
// Progress does not depend on which workgroups are resident: a workgroup
// owns a first-product tile only once it has exchanged the tile's start
// word from 0 to 1, right before running it, and a second-product tile
// whose dependencies are not finished runs every first-product tile of its
// M-tile that nobody has started yet itself.  So it only ever waits for
// tiles that a running workgroup is computing, and those have no
// dependencies -- also beside another chained launch on another stream.
//
// Workspace ints after the single-product scheduler's nine: the finished-
// workgroup counter, a sticky error word, 8 per-XCD position counters, and
// from CH_DEP on one completion counter per M-tile, then from CH_ST on one
// start word per first-product tile (all zero on entry and on exit).
constexpr int CH_DONE = 10, CH_ERR = 11, CH_XCD = 16, CH_DEP = 64;
constexpr int CH_MAX_MT = 16384;                 // M-tiles a chained launch can track
constexpr int CH_ST = CH_DEP + CH_MAX_MT;
constexpr int CH_MAX_T1 = 65536;                 // first-product tiles it can track
constexpr unsigned long long CH_WAIT_TICKS = 100000000ull;   // 1 s of the 100 MHz clock

// M-tile of tile t of a row-tiled product with NB N-tiles, and tile of
// (M-tile mi, N-tile nbi) -- the band order of run_tile.
__device__ __forceinline__ int mtile_of(int t, int NB, int MT) {
  const int band = GM_BAND * NB;
  const int first = (t / band) * GM_BAND;
  return first + (t % band) % min(GM_BAND, MT - first);
}
__device__ __forceinline__ int tile_at(int mi, int nbi, int NB, int MT) {
  const int first = mi / GM_BAND * GM_BAND;
  return first * NB + (mi - first) + nbi * min(GM_BAND, MT - first);
}

template <typename T, bool GATHER, int W>
__global__ __launch_bounds__(Waves<W>::NT, 1) void gmm_chain_kernel(GmmArgs a1, GmmArgs a2) {
  constexpr int NT = Waves<W>::NT;
  __shared__ __attribute__((aligned(1024))) char smem[RING_BYTES];
  __shared__ GroupLds gl;
  __shared__ int s_next, s_cmd;
  __shared__ int g_idx[4];
  const int tid = threadIdx.x;
  const int ng = a1.G + a1.shared;
  load_groups(a1, gl);
  tile_prefix(ng, gl);
  const Space s1 = tile_space<FWD1, false>(a1, gl, &s_next);
  const Space s2 = tile_space<FWD2, false>(a2, gl, &s_next);
  const int MT = gl.pre[ng];
  const int total1 = s1.total, total = s1.total + s2.total;
  int* const ws = a1.cnt;
  int* const dep = ws + CH_DEP;
  int* const st = ws + CH_ST;
  const int nwg = gridDim.x;
  const int nx = (nwg % 8 == 0) ? 8 : 1;
  const int xcd = blockIdx.x % nx, wpx = nwg / nx;
  // thread 0: the XCD whose sequence this workgroup draws from -- its own,
  // then, once that is used up, the next XCD's (as in persistent_loop)
  int vx = xcd;
  auto draw = [&]() {
    return __hip_atomic_fetch_add(ws + CH_XCD + vx, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  };
  auto pos_of = [&](int k) {   // position of draw k of XCD vx, moving on when it is used up
    int c = (k / wpx) * nwg + vx * wpx + k % wpx;
    for (int tries = 1; c >= total && tries < nx; ++tries) {
      vx = (vx + 1) % nx;
      const int k2 = draw();
      c = (k2 / wpx) * nwg + vx * wpx + k2 % wpx;
    }
    return c;
  };
  auto take = [&](int t) {   // thread 0: start first-product tile t unless started
    return __hip_atomic_exchange(st + t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
  };
  int grab = 0;   // thread 0: the sequence index drawn for the claim after this one
  int pend = -1;  // thread 0: a claimed second-product position still waiting
  if (tid == 0) s_next = draw();
  for (;;) {
    // every wave is done with the ring; s_next holds the drawn index
    __syncthreads();
    if (tid == 0) {
      // what this workgroup runs next (s_cmd): a first-product tile it owns
      // (claimed, or unstarted and needed by its waiting second-product
      // tile), a second-product tile whose row tile is done, or total: done
      int cmd = total;
      for (;;) {
        if (pend < 0) {
          // claim: a second-product position, or a first-product tile
          // nobody has started (else draw again)
          int k = s_next, c;
          for (;;) {
            c = pos_of(k);
            if (c >= total || c >= total1 || take(c)) break;
            k = draw();
          }
          if (c >= total) break;
          grab = draw();   // the claim after this one
          if (c < total1) {
            cmd = c;
            break;
          }
          pend = c;
        }
        const int mi = mtile_of(pend - total1, s2.NBt, MT);
        if (__hip_atomic_load(dep + mi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < s1.NBt) {
          int steal = -1;
          for (int nbi = 0; nbi < s1.NBt && steal < 0; ++nbi) {
            const int t1 = tile_at(mi, nbi, s1.NBt, MT);
            if (__hip_atomic_load(st + t1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0 &&
                take(t1))
              steal = t1;
          }
          if (steal >= 0) {   // run it now; the second-product tile stays pending
            cmd = steal;
            break;
          }
          // every first-product tile of the row tile is running elsewhere
          const unsigned long long t0 = wall_clock64();
          while (__hip_atomic_load(dep + mi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                 s1.NBt) {
            if (wall_clock64() - t0 > CH_WAIT_TICKS) {   // only when calls share a workspace
              __hip_atomic_store(ws + CH_ERR, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
        }
        // acquire: this CU's caches drop lines that may predate the count
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        cmd = pend;
        pend = -1;
        break;
      }
      s_cmd = cmd;
    }
    __syncthreads();
    const int c = uniform(s_cmd);
    if (c >= total) break;
    auto drained = [&]() {
      if (tid == 0) s_next = grab;   // read after the next loop-top barrier
    };
    if (c >= total1) {
      run_row_tile<T, FWD2, false, false, W>(a2, gl, s2, c - total1, smem, g_idx, drained);
      continue;
    }
    run_row_tile<T, FWD1, GATHER, false, W, true>(a1, gl, s1, c, smem, g_idx, drained);
    // publish: the act rows were stored at device scope (write-through), so
    // once every wave's stores have completed the count can go out -- the
    // compiler's agent-scope release for such stores is this same wait.  (A
    // release fence would also write back the whole L2 of this XCD, which
    // measured 8% of the launch for the small config's short tiles; h13 is
    // read by later launches only.)
    wait_vm<0>();
    __syncthreads();
    if (tid == 0)
      __hip_atomic_fetch_add(dep + mtile_of(c, s1.NBt, MT), 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
  // the last workgroup to finish (every draw and every publish of the
  // others done) returns the counters to zero for the next call
  __syncthreads();
  if (tid == 0)   // release: this workgroup's publishes land before its count
    s_cmd = __hip_atomic_fetch_add(ws + CH_DONE, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
            nwg - 1;
  __syncthreads();
  if (s_cmd) {
    for (int i = tid; i < MT; i += NT)
      __hip_atomic_store(dep + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = tid; i < total1; i += NT)
      __hip_atomic_store(st + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid < 8) __hip_atomic_store(ws + CH_XCD + tid, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) __hip_atomic_store(ws + CH_DONE, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------- act recompute
// act[r, :] = swiglu_act(h13[r, :I], h13[r, I:]) for the rows [lo, hi):
// the routed window [offsets[g0], offsets[g0+G]) (clamped to R), or [0, n)
// without offsets.  One 16-byte chunk of act per thread and pass.
template <typename T>
__global__ __launch_bounds__(256) void swiglu_act_kernel(const T* __restrict__ h13,
                                                         T* __restrict__ act,
                                                         const int32_t* __restrict__ offsets,
                                                         int g0, int G, int n, int I) {
  constexpr int ES = Cfg<T>::ES, VEC = Cfg<T>::VEC;
  int lo = 0, hi = n;
  if (offsets != nullptr) {
    lo = min(max(offsets[g0], 0), n);
    hi = min(max(offsets[g0 + G], lo), n);
  }
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(h13, clamp_bytes((long long)n * 2 * I * ES));
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(act, out_bytes((long long)n * I * ES));
  const int cpr = I / VEC;   // chunks per act row
  const long long total = (long long)(hi - lo) * cpr;
  for (long long c = (long long)blockIdx.x * 256 + threadIdx.x; c < total;
       c += (long long)gridDim.x * 256) {
    const int row = lo + (int)(c / cpr), q = (int)(c % cpr);
    const uint32_t ge = (uint32_t)row * (uint32_t)(2 * I) + (uint32_t)(q * VEC);
    float g[VEC], u[VEC], v[VEC];
    unpack16(buf_load16(hr, ge * ES), g, T());
    unpack16(buf_load16(hr, (ge + (uint32_t)I) * ES), u, T());
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] = swiglu_act<T>(g[e], u[e]);
    buf_store16(ar, ((uint32_t)row * (uint32_t)I + (uint32_t)(q * VEC)) * ES, pack16(v, T()));
  }
}

// ---------------------------------------------------------------- host side

int grid_size() {
  const int n = moe_cu_count();
  return n >= 8 ? (n / 8) * 8 : n;
}

// Workgroup shape: 4 waves.  The 8-wave shape (bf16 only) passes every
// parity test but measured slower on the Pangu share (gate/up product 669
// against 648 us, layer step 4.35 against 4.15 ms) although a bare main-loop
// microbenchmark ran it 5-14% faster (a higher clock at the same cycles per
// K step); its epilogues take longer with half the columns per wave.
template <typename T, int MODE, bool GATHER>
constexpr int WAVES = 4;

template <typename T, int MODE, bool GATHER = false, bool LIGHT = false>
int launch(const GmmArgs& a, hipStream_t s, const char* what) {
  constexpr int W = WAVES<T, MODE, GATHER>;
  hipLaunchKernelGGL((gmm_kernel<T, MODE, GATHER, LIGHT, W>), dim3(grid_size()),
                     dim3(Waves<W>::NT), 0, s, a);
  return moe_check_launch(what);
}

// a0: for the second launch of a backward call, the first launch's gradient
// product (its leading tiles beyond the first launch's share run here);
// M = 0 otherwise
template <int M1, int M2>
int launch_pair(int dt, const GmmArgs& a1, const GmmArgs& a2, const GmmArgs& a0, hipStream_t s,
                const char* what) {
  if (dt == MOE_BF16)
    hipLaunchKernelGGL((gmm_pair_kernel<bf16_t, M1, M2, WAVES<bf16_t, M1, false>>),
                       dim3(grid_size()), dim3(Waves<WAVES<bf16_t, M1, false>>::NT), 0, s, a1,
                       a2, a0);
  else
    hipLaunchKernelGGL((gmm_pair_kernel<float, M1, M2, 4>), dim3(grid_size()),
                       dim3(Waves<4>::NT), 0, s, a1, a2, a0);
  return moe_check_launch(what);
}

template <bool GATHER>
int launch_chain(int dt, const GmmArgs& a1, const GmmArgs& a2, hipStream_t s, const char* what) {
  constexpr int W = WAVES<bf16_t, FWD1, GATHER>;
  if (GATHER || dt == MOE_BF16)
    hipLaunchKernelGGL((gmm_chain_kernel<bf16_t, GATHER, W>), dim3(grid_size()),
                       dim3(Waves<W>::NT), 0, s, a1, a2);
  else
    hipLaunchKernelGGL((gmm_chain_kernel<float, false, 4>), dim3(grid_size()),
                       dim3(Waves<4>::NT), 0, s, a1, a2);
  return moe_check_launch(what);
}

// light: launch the build with the per-fragment-count loops (row-tiled bf16
// modes), for calls whose groups average at most half a tile of rows
template <int MODE>
int launch_dt(int dt, const GmmArgs& a, hipStream_t s, const char* what, bool light = false) {
  if constexpr (MODE != DW) {
    if (light && dt == MOE_BF16) {
      if constexpr (MODE == FWD1)
        if (a.gather != nullptr) return launch<bf16_t, MODE, true, true>(a, s, what);
      return launch<bf16_t, MODE, false, true>(a, s, what);
    }
  }
  if constexpr (MODE == FWD1 || MODE == DW)
    if (a.gather != nullptr) return launch<bf16_t, MODE, true>(a, s, what);   // bf16 only
  return dt == MOE_BF16 ? launch<bf16_t, MODE>(a, s, what) : launch<float, MODE>(a, s, what);
}

// Groups of a call that average at most half a 256-row tile: most of their
// tiles are mostly padding (DeepSeek-like routing over many experts).
bool small_groups(int G, int R) { return G > 0 && (long long)R <= (long long)G * (BM / 2); }

// Checks of a row gather from the token matrix x [T, H] (recompute variant).
int gather_checks(const char* fn, int dt, const void* x, const int32_t* src_token, int T, int H) {
  if (dt != MOE_BF16)
    return moe_fail(MOE_ERR_UNSUPPORTED, "%s: the row gather is built for bf16 only", fn);
  MOE_TRY(moe_need_nonneg(T, fn, "T"));
  MOE_TRY(moe_need_ptr(x, fn, "x"));
  MOE_TRY(moe_need_ptr(src_token, fn, "src_token", 4));
  if ((long long)T * H * 2 >= 0x80000000LL)
    return moe_fail(MOE_ERR_UNSUPPORTED, "%s: x of %d x %d bf16 is 2 GiB or more", fn, T, H);
  return MOE_OK;
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

// 9 scheduler counters, the forward chain's counters, per-M-tile counters and
// start words
constexpr size_t WS_BYTES = (size_t)(CH_ST + CH_MAX_T1) * 4;

// Attach the scheduler workspace (NULL: static tile order).
int attach_ws(GmmArgs& a, void* ws, size_t ws_bytes, const char* fn) {
  if (ws == nullptr) return MOE_OK;
  MOE_TRY(moe_need_ptr(ws, fn, "ws", 256));
  if (ws_bytes < WS_BYTES)
    return moe_fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes,
                    WS_BYTES);
  a.cnt = (int*)ws;
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

extern "C" size_t moe_gmm_workspace_bytes(void) { return WS_BYTES; }

namespace {

// Forward; gather != NULL: FWD1's routed rows are x[gather[r]] (xp is x).
int fwd_impl(const char* fn, const void* xp, const int32_t* gather, int gather_rows,
             const int32_t* offsets, int g0, int G, int R, int dt, int H, int I, const void* w13,
             const void* w2, void* h13, void* act, void* yp, const moe_shared_expert* sh,
             void* ws, size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(gmm_checks(fn, offsets, g0, G, R, dt, H, I, sh));
  if (G > 0 && R > 0) {
    MOE_TRY(moe_need_ptr(xp, fn, gather ? "x" : "xp"));
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
  MOE_TRY(attach_ws(a, ws, ws_bytes, fn));
  // FWD1: h13 = X . W13^T (N = 2I as I gate/up pairs, K = H)
  a.N = 2 * I; a.K = H; a.I = I;
  a.X = xp; a.ldx = H;
  a.gather = gather; a.gather_rows = gather_rows;
  a.W = w13; a.ldw = H; a.w_gs = 2LL * I * H;
  a.C = h13; a.ldc = 2 * I;
  a.C2 = act; a.ldc2 = I;
  if (use_sh) { a.sX = sh->x; a.sW = sh->w13; a.sC = sh->h13; a.sC2 = sh->act; }
  // FWD2: yp = act . W2^T (N = H, K = I)
  GmmArgs a2 = a;
  a2.gather = nullptr;
  a2.N = H; a2.K = I;
  a2.X = act; a2.ldx = I;
  a2.W = w2; a2.ldw = I; a2.w_gs = (long long)H * I;
  a2.C = yp; a2.ldc = H;
  a2.C2 = nullptr;
  if (use_sh) { a2.sX = sh->act; a2.sW = sh->w2; a2.sC = sh->y; a2.sC2 = nullptr; }
  const bool light = small_groups(a.G, R);
  // one chained launch where the workspace is there, the row tiles fit its
  // counters (a group adds at most one partial tile) and the groups are not
  // small ones (their light builds run as two launches)
  const long long mt_max = ((long long)R + BM - 1) / BM + a.G + ((long long)a.shT + BM - 1) / BM;
  const long long nb1 = (I + BN / 2 - 1) / (BN / 2);
  if (a.cnt != nullptr && !light && mt_max <= CH_MAX_MT && mt_max * nb1 <= CH_MAX_T1)
    return gather ? launch_chain<true>(dt, a, a2, s, fn) : launch_chain<false>(dt, a, a2, s, fn);
  MOE_TRY(launch_dt<FWD1>(dt, a, s, fn, light));
  return launch_dt<FWD2>(dt, a2, s, fn, light);
}

}  // namespace

extern "C" int moe_grouped_gemm_fwd(const void* xp, const int32_t* offsets, int g0, int G, int R,
                                    int dt, int H, int I, const void* w13, const void* w2,
                                    void* h13, void* act, void* yp,
                                    const moe_shared_expert* sh, void* ws, size_t ws_bytes,
                                    moe_stream_t stream) {
  return fwd_impl("moe_grouped_gemm_fwd", xp, nullptr, 0, offsets, g0, G, R, dt, H, I, w13, w2,
                  h13, act, yp, sh, ws, ws_bytes, stream);
}

extern "C" int moe_grouped_gemm_fwd_gather(const void* x, const int32_t* src_token, int T,
                                           const int32_t* offsets, int g0, int G, int R, int dt,
                                           int H, int I, const void* w13, const void* w2,
                                           void* h13, void* act, void* yp,
                                           const moe_shared_expert* sh, void* ws,
                                           size_t ws_bytes, moe_stream_t stream) {
  const char* fn = "moe_grouped_gemm_fwd_gather";
  MOE_TRY(gather_checks(fn, dt, x, src_token, T, H));
  return fwd_impl(fn, x, src_token, T, offsets, g0, G, R, dt, H, I, w13, w2, h13, act, yp, sh,
                  ws, ws_bytes, stream);
}

namespace {

int dx_checks(const char* fn, const void* dyp, const int32_t* offsets, int g0, int G, int R,
              int dt, int H, int I, const void* w13, const void* w2, const void* h13, void* dh13,
              void* dxp, const moe_shared_expert* sh) {
  MOE_TRY(gmm_checks(fn, offsets, g0, G, R, dt, H, I, sh));
  if (G > 0 && R > 0) {
    MOE_TRY(moe_need_ptr(dyp, fn, "dyp"));
    MOE_TRY(moe_need_ptr(w13, fn, "w13"));
    MOE_TRY(moe_need_ptr(w2, fn, "w2"));
    MOE_TRY(moe_need_ptr(h13, fn, "h13"));
    MOE_TRY(moe_need_ptr(dh13, fn, "dh13"));
    MOE_TRY(moe_need_ptr(dxp, fn, "dxp"));
  }
  if (sh && sh->T > 0) {
    MOE_TRY(moe_need_ptr(sh->dy, fn, "shared.dy"));
    MOE_TRY(moe_need_ptr(sh->w13, fn, "shared.w13"));
    MOE_TRY(moe_need_ptr(sh->w2, fn, "shared.w2"));
    MOE_TRY(moe_need_ptr(sh->h13, fn, "shared.h13"));
    MOE_TRY(moe_need_ptr(sh->dh13, fn, "shared.dh13"));
    MOE_TRY(moe_need_ptr(sh->dx, fn, "shared.dx"));
  }
  return MOE_OK;
}

// DX1: dact = dyp . W2 (W2 stored [K=H][N=I]), SwiGLU backward into dh13
void dx1_args(GmmArgs& a, const void* dyp, int H, int I, const void* w2, const void* h13,
              void* dh13, const moe_shared_expert* sh, bool use_sh) {
  a.N = I; a.K = H; a.I = I;
  a.X = dyp; a.ldx = H;
  a.W = w2; a.ldw = I; a.w_gs = (long long)H * I;
  a.C = dh13; a.ldc = 2 * I;
  a.aux = h13; a.ldaux = 2 * I;
  if (use_sh) { a.sX = sh->dy; a.sW = sh->w2; a.sC = sh->dh13; a.sAux = sh->h13; }
}

// DX2: dxp = dh13 . W13 (W13 stored [K=2I][N=H])
void dx2_args(GmmArgs& a, int H, int I, const void* w13, const void* dh13, void* dxp,
              const moe_shared_expert* sh, bool use_sh) {
  a.N = H; a.K = 2 * I; a.I = I;
  a.X = dh13; a.ldx = 2 * I;
  a.W = w13; a.ldw = H; a.w_gs = 2LL * I * H;
  a.C = dxp; a.ldc = H;
  a.aux = nullptr;
  if (use_sh) { a.sX = sh->dh13; a.sW = sh->w13; a.sC = sh->dx; a.sAux = nullptr; }
}

// dW2[e] [H,I] = dyp_e^T . act_e
void dw2_args(GmmArgs& a, const void* dyp, const void* act, int H, int I, void* dw2,
              const moe_shared_expert* sh, bool use_sh) {
  a.M = H; a.N = I; a.I = I;
  a.X = dyp; a.ldx = H;
  a.W = act; a.ldw = I;
  a.C = dw2; a.ldc = I; a.c_gs = (long long)H * I;
  if (use_sh) { a.sX = sh->dy; a.sW = sh->act; a.sC = sh->dw2; }
}

// dW13[e] [2I,H] = dh13_e^T . xp_e
void dw13_args(GmmArgs& a, const void* dh13, const void* xp, int H, int I, void* dw13,
               const moe_shared_expert* sh, bool use_sh) {
  a.M = 2 * I; a.N = H; a.I = I;
  a.X = dh13; a.ldx = 2 * I;
  a.W = xp; a.ldw = H;
  a.C = dw13; a.ldc = H; a.c_gs = 2LL * I * H;
  if (use_sh) { a.sX = sh->dh13; a.sW = sh->x; a.sC = sh->dw13; }
}

}  // namespace

extern "C" int moe_grouped_gemm_bwd_dx(const void* dyp, const int32_t* offsets, int g0, int G,
                                       int R, int dt, int H, int I, const void* w13,
                                       const void* w2, const void* h13, void* dh13, void* dxp,
                                       const moe_shared_expert* sh, void* ws, size_t ws_bytes,
                                       moe_stream_t stream) {
  const char* fn = "moe_grouped_gemm_bwd_dx";
  MOE_TRY(dx_checks(fn, dyp, offsets, g0, G, R, dt, H, I, w13, w2, h13, dh13, dxp, sh));
  const bool use_sh = sh && sh->T > 0;
  if (!use_sh && (G == 0 || R == 0)) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  GmmArgs a = base_args(offsets, g0, (R > 0) ? G : 0, R, sh);
  MOE_TRY(attach_ws(a, ws, ws_bytes, fn));
  dx1_args(a, dyp, H, I, w2, h13, dh13, sh, use_sh);
  MOE_TRY(launch_dt<DX1>(dt, a, s, fn, small_groups(a.G, R)));
  dx2_args(a, H, I, w13, dh13, dxp, sh, use_sh);
  return launch_dt<DX2>(dt, a, s, fn, small_groups(a.G, R));
}

namespace {

// Weight gradients; gather != NULL: dW13's routed K rows of xp are
// x[gather[r]] (xp is x); h13 != NULL: act (and the shared expert's act) is
// first recomputed from h13.
int dw_impl(const char* fn, const void* xp, const int32_t* gather, int gather_rows,
            const void* h13, void* act, const void* dyp, const void* dh13,
            const int32_t* offsets, int g0, int G, int R, int dt, int H, int I, void* dw13,
            void* dw2, const moe_shared_expert* sh, void* ws, size_t ws_bytes,
            moe_stream_t stream) {
  MOE_TRY(gmm_checks(fn, offsets, g0, G, R, dt, H, I, sh));
  if (G > 0) {
    MOE_TRY(moe_need_ptr(dw13, fn, "dw13"));
    MOE_TRY(moe_need_ptr(dw2, fn, "dw2"));
    if (R > 0) {
      if (h13) MOE_TRY(moe_need_ptr(h13, fn, "h13"));
      MOE_TRY(moe_need_ptr(xp, fn, gather ? "x" : "xp"));
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
      if (h13) MOE_TRY(moe_need_ptr(sh->h13, fn, "shared.h13"));
    }
  }
  if (!use_sh && G == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (h13) {
    // act of the routed window and of the shared expert, from h13
    const int grid = 4 * grid_size();
    if (G > 0 && R > 0) {
      hipLaunchKernelGGL(swiglu_act_kernel<bf16_t>, dim3(grid), dim3(256), 0, s,
                         (const bf16_t*)h13, (bf16_t*)act, offsets, g0, G, R, I);
      MOE_TRY(moe_check_launch(fn));
    }
    if (use_sh && sh->T > 0) {
      hipLaunchKernelGGL(swiglu_act_kernel<bf16_t>, dim3(grid), dim3(256), 0, s,
                         (const bf16_t*)sh->h13, (bf16_t*)sh->act, nullptr, 0, 0, sh->T, I);
      MOE_TRY(moe_check_launch(fn));
    }
  }
  GmmArgs a = base_args(offsets, g0, G, R, sh);
  MOE_TRY(attach_ws(a, ws, ws_bytes, fn));
  a.shared = use_sh ? 1 : 0;   // an empty shared expert still gets zero gradients
  a.shT = use_sh ? sh->T : 0;
  dw2_args(a, dyp, act, H, I, dw2, sh, use_sh);
  MOE_TRY(launch_dt<DW>(dt, a, s, fn));
  dw13_args(a, dh13, xp, H, I, dw13, sh, use_sh);
  a.gather = gather; a.gather_rows = gather_rows;
  return launch_dt<DW>(dt, a, s, fn);
}

}  // namespace

extern "C" int moe_grouped_gemm_bwd_dw(const void* xp, const void* act, const void* dyp,
                                       const void* dh13, const int32_t* offsets, int g0, int G,
                                       int R, int dt, int H, int I, void* dw13, void* dw2,
                                       const moe_shared_expert* sh, void* ws, size_t ws_bytes,
                                       moe_stream_t stream) {
  return dw_impl("moe_grouped_gemm_bwd_dw", xp, nullptr, 0, nullptr, const_cast<void*>(act), dyp,
                 dh13, offsets, g0, G, R, dt, H, I, dw13, dw2, sh, ws, ws_bytes, stream);
}

// dX and dW of one call: two persistent launches, each holding one product of
// dX and one weight-gradient product that needs nothing from it --
// [dact + SwiGLU bwd | dW2], then [dX | dW13] (dW13 reads the dh13 the first
// launch wrote; the second launch also runs the leading dW2 tiles the first
// leaves to it) -- so that neither dX product ends in a partial round of its
// own; every output is the same bits as moe_grouped_gemm_bwd_dx followed by
// moe_grouped_gemm_bwd_dw.  Calls whose shapes the paired launches do not
// cover (an empty shared expert, no rows, the small-group build) take the
// two calls' launches instead.
extern "C" int moe_grouped_gemm_bwd(const void* xp, const void* act, const void* dyp,
                                    const int32_t* offsets, int g0, int G, int R, int dt, int H,
                                    int I, const void* w13, const void* w2, const void* h13,
                                    void* dh13, void* dxp, void* dw13, void* dw2,
                                    const moe_shared_expert* sh, void* ws, size_t ws_bytes,
                                    moe_stream_t stream) {
  const char* fn = "moe_grouped_gemm_bwd";
  MOE_TRY(dx_checks(fn, dyp, offsets, g0, G, R, dt, H, I, w13, w2, h13, dh13, dxp, sh));
  if (G > 0) {
    MOE_TRY(moe_need_ptr(dw13, fn, "dw13"));
    MOE_TRY(moe_need_ptr(dw2, fn, "dw2"));
    if (R > 0) {
      MOE_TRY(moe_need_ptr(xp, fn, "xp"));
      MOE_TRY(moe_need_ptr(act, fn, "act"));
    }
  }
  const bool sh_rows = sh && sh->T > 0;
  const bool sh_grads = sh && sh->T >= 0 && (sh->dw13 || sh->dw2);
  if (sh_grads) {
    MOE_TRY(moe_need_ptr(sh->dw13, fn, "shared.dw13"));
    MOE_TRY(moe_need_ptr(sh->dw2, fn, "shared.dw2"));
    if (sh_rows) {
      MOE_TRY(moe_need_ptr(sh->x, fn, "shared.x"));
      MOE_TRY(moe_need_ptr(sh->act, fn, "shared.act"));
    }
  }
  // paired launches: both products on the same window (the shared expert,
  // if any, has rows and gets its gradients), and the plain build
  const bool paired = (G > 0 && R > 0 && !small_groups(G, R) && (!sh || (sh_rows && sh_grads))) ||
                      (G == 0 && sh_rows && sh_grads);
  if (!paired) {
    MOE_TRY(moe_grouped_gemm_bwd_dx(dyp, offsets, g0, G, R, dt, H, I, w13, w2, h13, dh13, dxp, sh,
                                    ws, ws_bytes, stream));
    return moe_grouped_gemm_bwd_dw(xp, act, dyp, dh13, offsets, g0, G, R, dt, H, I, dw13, dw2, sh,
                                   ws, ws_bytes, stream);
  }
  hipStream_t s = (hipStream_t)stream;
  GmmArgs a1 = base_args(offsets, g0, G, R, sh);
  MOE_TRY(attach_ws(a1, ws, ws_bytes, fn));
  GmmArgs a2 = a1;
  dx1_args(a1, dyp, H, I, w2, h13, dh13, sh, sh_rows);
  dw2_args(a2, dyp, act, H, I, dw2, sh, sh_rows);
  const GmmArgs none = {};
  MOE_TRY((launch_pair<DX1, DW>(dt, a1, a2, none, s, fn)));
  const GmmArgs a0 = a2;
  dx2_args(a1, H, I, w13, dh13, dxp, sh, sh_rows);
  dw13_args(a2, dh13, xp, H, I, dw13, sh, sh_rows);
  return launch_pair<DX2, DW>(dt, a1, a2, a0, s, fn);
}

extern "C" int moe_grouped_gemm_bwd_dw_recompute(const void* x, const int32_t* src_token, int T,
                                                 const void* h13, void* act, const void* dyp,
                                                 const void* dh13, const int32_t* offsets,
                                                 int g0, int G, int R, int dt, int H, int I,
                                                 void* dw13, void* dw2,
                                                 const moe_shared_expert* sh, void* ws,
                                                 size_t ws_bytes, moe_stream_t stream) {
  const char* fn = "moe_grouped_gemm_bwd_dw_recompute";
  MOE_TRY(gather_checks(fn, dt, x, src_token, T, H));
  if (h13 == nullptr) return moe_fail(MOE_ERR_INVALID_ARG, "%s: h13 is NULL", fn);
  return dw_impl(fn, x, src_token, T, h13, act, dyp, dh13, offsets, g0, G, R, dt, H, I, dw13,
                 dw2, sh, ws, ws_bytes, stream);
}


// ---------------------------------------------------------------- router products
// The fp32 router projection on the bf16 MFMA path (used for bf16 tokens):
// the fp32 factor is split into three bf16 parts (hi + mid + lo carry all 24
// mantissa bits), each part's product with the exact bf16 tokens is exact in
// fp32, and the K range is cut into S slices whose fp32 partial sums are
// added in fp64 by the caller, which keeps the result within a few fp32 ulps.

int moe_gmm_router_fwd(const void* x, const void* wg3s, float* partials, int T, int H, int E, int S,
                       hipStream_t s) {
  GmmArgs a = {};
  a.dense = 1; a.G = S; a.shT = T; a.R = T;
  a.N = E; a.K = 3 * (H / S); a.krep = 3;
  a.X = x; a.ldx = H; a.x_gs = H / S;
  a.W = wg3s; a.ldw = E; a.w_gs = 3LL * (H / S) * E;
  a.C = partials; a.ldc = E; a.c_gs = (long long)T * E; a.out_f32 = 1;
  return launch<bf16_t, DX2>(a, s, "moe_router_logits");
}

int moe_gmm_router_dx(const void* dlb, const void* wgb, void* dx, int T, int H, int E,
                      hipStream_t s) {
  GmmArgs a = {};
  a.dense = 1; a.G = 1; a.shT = T; a.R = T;
  a.N = H; a.K = E;
  a.X = dlb; a.ldx = E;
  a.W = wgb; a.ldw = E;
  a.C = dx; a.ldc = H;
  return launch<bf16_t, FWD2>(a, s, "moe_router_logits_bwd(dx)");
}

int moe_gmm_router_dwg(const void* x, const void* dl3s, float* partials, int T, int H, int E, int S,
                       hipStream_t s) {
  GmmArgs a = {};
  a.dense = 1; a.G = S; a.shT = 3 * (T / S); a.R = T;
  a.M = H; a.N = E; a.krep = 3;
  a.X = x; a.ldx = H; a.x_gs = (long long)(T / S) * H;
  a.W = dl3s; a.ldw = E; a.w_gs = 3LL * (T / S) * E;
  a.C = partials; a.ldc = E; a.c_gs = (long long)H * E; a.out_f32 = 1;
  return launch<bf16_t, DW>(a, s, "moe_router_logits_bwd(dwg)");
}
